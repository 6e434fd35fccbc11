// tau_rows.hip -- row-wise 1.5-entmax threshold and probabilities on a
// materialised fp32 score matrix (the HBM-bound row kernel).
//
// Rows up to 8192 wide: single-wave workgroups, as many as stay resident,
// each looping over its rows.  A row is read from HBM once into registers
// (128 values per lane at 8192 columns, which leaves room for three waves
// per SIMD, i.e. 12 rows in flight per CU).  Every reduction is a DPP wave
// reduction; there are no barriers.  Per row:
//   1. the maximum m;
//   2. a lower bound on tau from the 64 lane maxima, a subset of the row (a
//      threshold only rises as scores are added): Newton steps from m - 2,
//      which stay below the subset's threshold;
//   3. the scores above that bound, compacted into LDS (usually little more
//      than the support);
//   4. tau from those candidates by the hybrid Halley-bisection of "AdaSplash:
//      Adaptive Sparse Flash Attention" (summary, Approach), inside the
//      bracket [lower bound, m - 2/sqrt(n)] of "AdaSplash-2: Faster
//      Differentiable Sparse Attention" sec. 2.4 (score units), with an exact
//      finish: once the set {s > t} is the support, the normaliser restricted
//      to it is a quadratic in tau solved in closed form (the S0/S1/S2 form of
//      AdaSplash-2 appendix C.3);
//   5. P from the register copy, so HBM sees one read and one write per
//      element; the loads of the wave's next row are issued into the
//      registers as they free up.
// Rows up to 32768 wide (float4 access): a 256-thread workgroup holds the
// row in registers instead (tau_rows_block), so the refinement steps of a
// dense row never re-read it.  Wider rows take a 256-thread streaming kernel
// that reads the row three times (maximum, candidates above m - 2, output).
// While it compacts the candidates it also bins them (the histogram
// initialisation of AdaSplash-2 sec. 3.1, 64 left-edge bins): the histogram
// threshold tau_h brackets tau within one bin width, so the refinement starts
// from [tau_h, tau_h + h] instead of the whole [m - 2, m - 2/sqrt(n)].  That
// matters when a dense row overflows the LDS list and every refinement step
// re-reads the row.
//
// Other alpha in (1, 2] (AdaSplash-2 sec. 2.3; see AlphaMap) take the same
// structure with p = [(alpha-1)(s - tau)]_+^(1/(alpha-1)): the lower bound is
// the threshold of the lane maxima (the subset argument holds for every
// alpha), and tau comes from Newton steps from below on the candidates with
// a bisection guard (no closed form for general alpha).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "device_common.hpp"
#include "launch.hpp"
#include "row_solve.hpp"

namespace entmax {
namespace {

using namespace rows;

constexpr int kWaveCand = 2048;  // LDS candidates per wave
constexpr int kMaxDevices = 64;

// Loads of one row into registers: chunk k of VEC rows is the float4 at
// column (64 k + lane) * 4, otherwise element 64 k + lane; entries at or past
// cols read -inf.  FULL: cols == 64 VPT, every chunk lies inside the row (no
// guards).
template <int VPT, bool VEC, bool FULL>
struct RowRegs {
    float v[VPT];

    __device__ __forceinline__ void load_chunk(const float* src, int k, int cols, int lane) {
        if constexpr (VEC) {
            const int pos = (k * kWave + lane) * 4;
            if constexpr (FULL) {
                const f32x4 q = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(src + pos));
#pragma unroll
                for (int e = 0; e < 4; ++e) v[4 * k + e] = q[e];
            } else {
                // chunks past the end re-read the last chunk that starts
                // inside the row (ld % 4 == 0, so it lies within the row's
                // ld span)
                const int last = ((cols - 1) / 4) * 4;
                const f32x4 q = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(src + min(pos, last)));
#pragma unroll
                for (int e = 0; e < 4; ++e) v[4 * k + e] = (pos + e < cols) ? q[e] : neg_inf();
            }
        } else {
            const int pos = k * kWave + lane;
            v[k] = (FULL || pos < cols) ? src[pos] : neg_inf();
        }
    }
    static constexpr int kChunks = VEC ? VPT / 4 : VPT;
};

// Rows up to 64 VPT wide, one wave per workgroup, each wave taking rows
// blockIdx.x, blockIdx.x + gridDim.x, ... (the grid is what stays resident,
// so no workgroup waits for a slot).  The row is held in registers (VPT
// values per lane) and read from HBM once; while the wave computes and
// stores the probabilities of one row, it issues the loads of its next row
// into the registers it has just used, so its slot keeps memory requests in
// flight through the store phase.  No barriers.  VEC: float4 accesses
// (ld % 4 == 0 and 16-byte aligned S / P).
template <int VPT, bool VEC, bool FULL, bool GEN>
__global__ __launch_bounds__(kWave, 3) void tau_rows_wave(const float* __restrict__ S,
                                                         float* __restrict__ P,
                                                         float* __restrict__ tau_out,
                                                         int64_t rows, int cols, int64_t ld,
                                                         AlphaMap am) {
    using Regs = RowRegs<VPT, VEC, FULL>;
    __shared__ float cand[kWaveCand + kWave];
    const int lane = threadIdx.x;
    int64_t row = blockIdx.x;
    if (row >= rows) return;
    Regs r;
    float* v = r.v;
#pragma unroll
    for (int k = 0; k < Regs::kChunks; ++k) r.load_chunk(S + row * ld, k, cols, lane);

    for (;;) {
        const float* src = S + row * ld;
        float mx = neg_inf();
#pragma unroll
        for (int k = 0; k < VPT; ++k) mx = fmaxf(mx, v[k]);
        const float m = wave_max_dpp(mx);

        float tau;
        if (m == neg_inf()) {
            tau = neg_inf();  // no active entry: P = 0
        } else {
            // Lower bound from the 64 lane maxima, a subset of the row (a
            // threshold only rises as scores are added).  The row's largest
            // scores mostly sit in different lanes, so the bound is close to
            // tau and few scores lie above it.
            float tlo;
            if constexpr (GEN) {
                const float n1 = wave_sum_dpp(mx > neg_inf() ? 1.0f : 0.0f);
                wave_tau_gen(m, n1, m - am.e, am, [&](float tt, RowSums& s) { accumulate_gen(s, mx, tt, am); },
                             &tlo);
            } else {
                tlo = wave_newton_lower(mx, m);
            }
            // The scores above it, compacted into LDS in register order.  The
            // comparisons of 8 registers are taken first, as wave masks, so
            // the scalar tests that skip registers with no candidate in any
            // lane do not wait on each comparison in turn; slots past the
            // list go to the lane's spare word.
            int n = 0;
#pragma unroll
            for (int k0 = 0; k0 < VPT; k0 += 8) {
                uint64_t b[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) b[j] = __ballot(v[k0 + j] > tlo);
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    if (b[j] != 0) {
                        const int slot = min(n + lanes_below(b[j]), kWaveCand + lane);
                        if (v[k0 + j] > tlo) cand[slot] = v[k0 + j];
                        n += __popcll(b[j]);
                    }
                }
            }
            if constexpr (GEN) {
                if (n <= kWaveCand) {
                    tau = wave_tau_gen(m, (float)n, tlo, am, [&](float tt, RowSums& s) {
                        for (int i = lane; i < n; i += kWave) accumulate_gen(s, cand[i], tt, am);
                    }, nullptr);
                } else {
                    tau = wave_tau_gen(m, (float)n, tlo, am, [&](float tt, RowSums& s) {
                        for (int pos = lane; pos < cols; pos += kWave) accumulate_gen(s, src[pos], tt, am);
                    }, nullptr);
                }
            } else if (n <= kWaveCand) {
                tau = wave_tau(m, (float)n, tlo, [&](float tt, RowSums& s) {
                    for (int i = lane; i < n; i += kWave) accumulate(s, cand[i], tt, m);
                });
            } else {
                // more candidates than the LDS list (near-constant rows):
                // sweep the row in memory each iteration (the register copy
                // would be pinned twice over by the loop)
                tau = wave_tau(m, (float)n, tlo, [&](float tt, RowSums& s) {
                    for (int pos = lane; pos < cols; pos += kWave) accumulate(s, src[pos], tt, m);
                });
            }
        }

        if (lane == 0) tau_out[row] = tau;
        // an opaque copy of the lane index for the addresses and bounds
        // below: keeps the compiler from hoisting them out of the row loop,
        // which would pin a register or a mask for each chunk
        int li = lane;
        asm volatile("" : "+v"(li));
        const int64_t next = row + gridDim.x;
        const bool more = next < rows;
        const float* nsrc = S + (more ? next : row) * ld;
        if (P == nullptr) {
            if (!more) break;
#pragma unroll
            for (int k = 0; k < Regs::kChunks; ++k) r.load_chunk(nsrc, k, cols, li);
            row = next;
            continue;
        }
        float* dst = P + row * ld;
        const float h = -0.5f * tau;
        auto pr = [&](float x) -> float {
            if constexpr (GEN) return am.p(x, tau);
            else return prob_h(x, h);
        };
#pragma unroll
        for (int k = 0; k < Regs::kChunks; ++k) {
            if constexpr (VEC) {
                const int pos = (k * kWave + li) * 4;
                f32x4 q;
#pragma unroll
                for (int e = 0; e < 4; ++e) q[e] = pr(v[4 * k + e]);
                if (FULL || pos + 3 < cols) {
                    __builtin_nontemporal_store(q, reinterpret_cast<f32x4*>(dst + pos));
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (pos + e < cols) dst[pos + e] = q[e];
                }
            } else {
                const int pos = k * kWave + li;
                if (FULL || pos < cols) dst[pos] = pr(v[k]);
            }
            if (more) r.load_chunk(nsrc, k, cols, li);
        }
        if (!more) break;
        row = next;
    }
}

// Rows of 64 VPT < cols <= 256 VPT (float4 access): a 256-thread workgroup
// holds the row in registers, VPT values per thread, so HBM sees one read and
// one write per element however many refinement steps the row needs (a dense
// row's candidates overflow any LDS list).  Every Halley-bisection step
// visits the registers, from the plain bracket: a step over registers costs
// less than the histogram's LDS atomic per score (measured on dense rows of
// 32768: 0.196 ms for 2048 rows from the plain bracket, 0.259 ms with the
// histogram first).  Three rows per CU in flight at VPT = 64, two at 128
// (256 KB per CU, more than HBM needs in flight).
// FULL: cols == 256 VPT, no bounds on the accesses.
template <int VPT, bool FULL, bool GEN>
__global__ __launch_bounds__(kThreads, (VPT <= 64 ? 3 : 2)) void tau_rows_block(const float* __restrict__ S,
                                                             float* __restrict__ P,
                                                             float* __restrict__ tau_out, int cols,
                                                             int64_t ld, AlphaMap am) {
    static_assert(VPT % 4 == 0, "float4 chunks");
    __shared__ float red[2][kWaves][6];
    __shared__ float mbuf[kWaves];
    const int t = threadIdx.x;
    const int64_t row = blockIdx.x;
    const float* src = S + row * ld;
    constexpr int kCh = VPT / 4;
    // chunk k of the thread is the float4 at column (256 k + t) * 4; chunks
    // past the end re-read the last chunk that starts inside the row
    const int last = ((cols - 1) / 4) * 4;
    float v[VPT];
#pragma unroll
    for (int k = 0; k < kCh; ++k) {
        const int pos = (k * kThreads + t) * 4;
        const f32x4 q = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(src + (FULL ? pos : min(pos, last))));
#pragma unroll
        for (int e = 0; e < 4; ++e) v[4 * k + e] = (FULL || pos + e < cols) ? q[e] : neg_inf();
    }
    float mx = neg_inf();
#pragma unroll
    for (int k = 0; k < VPT; ++k) mx = fmaxf(mx, v[k]);
    const float m = block_max(mx, mbuf);

    float tau;
    if (m == neg_inf()) {
        tau = neg_inf();
    } else {
        // (cols bounds the active count from above, which keeps the upper
        // bracket end m - 2/sqrt(n) valid).  Each step reads the registers
        // through an opaque copy: otherwise the compiler hoists the
        // step-invariant part of every term (x - m) out of the loop and keeps
        // a second copy of the row, which spills.
        if constexpr (GEN) {
            tau = refine_tau_gen(m, (float)cols, am, [&](float tt, RowSums& s) {
#pragma unroll
                for (int k = 0; k < VPT; ++k) {
                    float x = v[k];
                    asm volatile("" : "+v"(x));
                    accumulate_gen(s, x, tt, am);
                }
            }, red);
        } else {
            tau = refine_tau(m, (float)cols, [&](float tt, RowSums& s) {
#pragma unroll
                for (int k = 0; k < VPT; ++k) {
                    float x = v[k];
                    asm volatile("" : "+v"(x));
                    accumulate(s, x, tt, m);
                }
            }, red);
        }
    }
    if (t == 0) tau_out[row] = tau;
    if (P == nullptr) return;
    float* dst = P + row * ld;
    const float h = -0.5f * tau;
    // an opaque copy of the thread index: the bounds below are not the
    // loads' bounds kept alive through the refinement (one mask per chunk)
    int ti = t;
    asm volatile("" : "+v"(ti));
#pragma unroll
    for (int k = 0; k < kCh; ++k) {
        const int pos = (k * kThreads + ti) * 4;
        f32x4 q;
#pragma unroll
        for (int e = 0; e < 4; ++e) q[e] = GEN ? am.p(v[4 * k + e], tau) : prob_h(v[4 * k + e], h);
        if (FULL || pos + 3 < cols) {
            __builtin_nontemporal_store(q, reinterpret_cast<f32x4*>(dst + pos));
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (pos + e < cols) dst[pos + e] = q[e];
        }
    }
}

// Any width: the row is streamed from global memory (L2-resident after the
// first pass for moderate widths).
template <bool GEN>
__global__ __launch_bounds__(kThreads) void tau_rows_stream(const float* __restrict__ S,
                                                           float* __restrict__ P,
                                                           float* __restrict__ tau_out,
                                                           int64_t cols, int64_t ld, AlphaMap am,
                                                           int use_hist) {
    __shared__ float cand[kCandCap];
    __shared__ float red[2][kWaves][6];
    __shared__ float mbuf[kWaves];
    __shared__ int wcnt[kWaves];
    __shared__ int hist[kWaves][kHistBins];
    __shared__ float tauh_s;

    const int t = threadIdx.x, lane = t & (kWave - 1), w = wave_id();
    const int64_t row = blockIdx.x;
    const float* src = S + row * ld;
    for (int i = t; i < kWaves * kHistBins; i += kThreads) (&hist[0][0])[i] = 0;

    float mx = neg_inf();
    for (int64_t pos = t; pos < cols; pos += kThreads) mx = fmaxf(mx, src[pos]);
    const float m = block_max(mx, mbuf);

    float tau;
    if (m == neg_inf()) {
        tau = neg_inf();
    } else {
        const float lo0 = GEN ? m - am.e : m - 2.0f;  // lower bracket end
        // Compact candidates in chunk order; placement is deterministic.
        int filled = 0;  // candidates seen so far (may exceed the capacity)
        const int64_t chunks = (cols + kThreads - 1) / kThreads;
        for (int64_t c = 0; c < chunks; ++c) {
            const int64_t pos = c * kThreads + t;
            const float x = (pos < cols) ? src[pos] : neg_inf();
            const bool is_c = x > lo0;
            const uint64_t b = __ballot(is_c);
            if (lane == 0) wcnt[w] = __popcll(b);
            __syncthreads();
            int base = filled, tot = 0;
#pragma unroll
            for (int i = 0; i < kWaves; ++i) {
                base += (i < w) ? wcnt[i] : 0;
                tot += wcnt[i];
            }
            const int slot = base + lanes_below(b);
            if (is_c && slot < kCandCap) cand[slot] = x;
            if (is_c && use_hist) atomicAdd(&hist[w][hist_bin(x, m, am.am1)], 1);
            filled += tot;
            __syncthreads();
        }
        // histogram bracket [tau_h, tau_h + 1/(B (alpha - 1))], widened by a
        // rounding margin (bins come from fp32 z)
        float blo = neg_inf(), bhi = __builtin_inff();
        if (use_hist) {
            if (w == 0) {
                int cnt = 0;
#pragma unroll
                for (int k = 0; k < kWaves; ++k) cnt += hist[k][lane];
                const float th = hist_tau(cnt, m, am);
                if (lane == 0) tauh_s = th;
            }
            __syncthreads();
            const float th = tauh_s;
            const float marg = 1e-6f * fmaxf(1.0f, fabsf(th));
            blo = th - marg;
            bhi = th + am.e / (float)kHistBins + marg;
        }
        if constexpr (GEN) {
            if (filled <= kCandCap) {
                tau = refine_tau_gen(m, (float)filled, am, [&](float tt, RowSums& s) {
                    for (int i = t; i < filled; i += kThreads) accumulate_gen(s, cand[i], tt, am);
                }, red, blo, bhi);
            } else {
                tau = refine_tau_gen(m, (float)filled, am, [&](float tt, RowSums& s) {
                    for (int64_t pos = t; pos < cols; pos += kThreads) accumulate_gen(s, src[pos], tt, am);
                }, red, blo, bhi);
            }
        } else if (filled <= kCandCap) {
            tau = refine_tau(
                m, (float)filled,
                [&](float tt, RowSums& s) {
                    for (int i = t; i < filled; i += kThreads) accumulate(s, cand[i], tt, m);
                },
                red, blo, bhi);
        } else {
            tau = refine_tau(
                m, (float)filled,
                [&](float tt, RowSums& s) {
                    for (int64_t pos = t; pos < cols; pos += kThreads) accumulate(s, src[pos], tt, m);
                },
                red, blo, bhi);
        }
    }
    if (t == 0) tau_out[row] = tau;
    if (P == nullptr) return;
    float* dst = P + row * ld;
    for (int64_t pos = t; pos < cols; pos += kThreads) dst[pos] = GEN ? am.p(src[pos], tau) : prob(src[pos], tau);
}

template <int VPT, bool VEC, bool FULL, bool GEN>
hipError_t launch_wave_inst(const float* S, float* P, float* tau, int64_t rows, int64_t cols,
                       int64_t ld, const AlphaMap& am, hipStream_t stream) {
    // as many waves as stay resident at once (each loops over its rows)
    static int per_cu[kMaxDevices] = {};
    static int cus[kMaxDevices] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    if (per_cu[dev] == 0) {
        int nb = 0, nc = 0;
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, tau_rows_wave<VPT, VEC, FULL, GEN>, kWave, 0);
        if (e != hipSuccess) return e;
        e = hipDeviceGetAttribute(&nc, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return e;
        cus[dev] = nc;
        per_cu[dev] = nb > 0 ? nb : 1;
    }
    const int64_t blocks = std::min<int64_t>(rows, (int64_t)per_cu[dev] * cus[dev]);
    hipLaunchKernelGGL((tau_rows_wave<VPT, VEC, FULL, GEN>), dim3((unsigned)blocks), dim3(kWave), 0, stream, S,
                       P, tau, rows, (int)cols, ld, am);
    return hipGetLastError();
}

template <int VPT, bool VEC, bool GEN>
hipError_t launch_wave(const float* S, float* P, float* tau, int64_t rows, int64_t cols,
                       int64_t ld, const AlphaMap& am, hipStream_t stream) {
    if (cols == VPT * kWave) return launch_wave_inst<VPT, VEC, true, GEN>(S, P, tau, rows, cols, ld, am, stream);
    return launch_wave_inst<VPT, VEC, false, GEN>(S, P, tau, rows, cols, ld, am, stream);
}

template <bool GEN>
hipError_t launch_rows(const float* S, float* P, float* tau, int64_t rows, int64_t cols, int64_t ld,
                       const AlphaMap& am, int use_hist, hipStream_t stream) {
    const bool vec = (ld % 4 == 0) && ((uintptr_t)S % 16 == 0) &&
                     (P == nullptr || (uintptr_t)P % 16 == 0);
    if (vec) {
        if (cols <= 8 * kWave) return launch_wave<8, true, GEN>(S, P, tau, rows, cols, ld, am, stream);
        if (cols <= 16 * kWave) return launch_wave<16, true, GEN>(S, P, tau, rows, cols, ld, am, stream);
        if (cols <= 32 * kWave) return launch_wave<32, true, GEN>(S, P, tau, rows, cols, ld, am, stream);
        if (cols <= 64 * kWave) return launch_wave<64, true, GEN>(S, P, tau, rows, cols, ld, am, stream);
        if (cols <= 128 * kWave) return launch_wave<128, true, GEN>(S, P, tau, rows, cols, ld, am, stream);
        if (cols <= 128 * kThreads) {
            const dim3 grid((unsigned)rows), block(kThreads);
            if (cols == 64 * kThreads)
                hipLaunchKernelGGL((tau_rows_block<64, true, GEN>), grid, block, 0, stream, S, P, tau, (int)cols, ld,
                                   am);
            else if (cols < 64 * kThreads)
                hipLaunchKernelGGL((tau_rows_block<64, false, GEN>), grid, block, 0, stream, S, P, tau, (int)cols,
                                   ld, am);
            else if (cols == 128 * kThreads)
                hipLaunchKernelGGL((tau_rows_block<128, true, GEN>), grid, block, 0, stream, S, P, tau, (int)cols,
                                   ld, am);
            else
                hipLaunchKernelGGL((tau_rows_block<128, false, GEN>), grid, block, 0, stream, S, P, tau, (int)cols,
                                   ld, am);
            return hipGetLastError();
        }
    } else {
        if (cols <= 8 * kWave) return launch_wave<8, false, GEN>(S, P, tau, rows, cols, ld, am, stream);
        if (cols <= 16 * kWave) return launch_wave<16, false, GEN>(S, P, tau, rows, cols, ld, am, stream);
        if (cols <= 32 * kWave) return launch_wave<32, false, GEN>(S, P, tau, rows, cols, ld, am, stream);
        if (cols <= 64 * kWave) return launch_wave<64, false, GEN>(S, P, tau, rows, cols, ld, am, stream);
    }
    hipLaunchKernelGGL(tau_rows_stream<GEN>, dim3((unsigned)rows), dim3(kThreads), 0, stream, S, P,
                       tau, cols, ld, am, use_hist);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_tau_rows(const float* S, float* P, float* tau, int64_t rows, int64_t cols,
                           int64_t ld, float alpha, int use_hist, hipStream_t stream) {
    const AlphaMap am = make_alpha_map(alpha);
    if (alpha == 1.5f) return launch_rows<false>(S, P, tau, rows, cols, ld, am, use_hist, stream);
    return launch_rows<true>(S, P, tau, rows, cols, ld, am, use_hist, stream);
}

}  // namespace entmax
