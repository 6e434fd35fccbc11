// tau_rows.hip -- row-wise 1.5-entmax threshold and probabilities on a
// materialised fp32 score matrix (the HBM-bound row kernel).
//
// One 256-thread workgroup per row.  The row is read from HBM once into
// registers, its maximum m is reduced across the workgroup, and the scores
// above m - 2 (the lower bracket end of "AdaSplash-2: Faster Differentiable
// Sparse Attention" sec. 2.4 in score units; no score at or below it can carry
// weight) are compacted into LDS.  The threshold is then refined on those few
// candidates only with the hybrid Halley-bisection of "AdaSplash: Adaptive
// Sparse Flash Attention" (summary, Approach), safeguarded by the bracket
// [m - 2, m - 2/sqrt(n)], with an exact finish: when tau sits below the
// support, the support is {s > tau} and the normaliser restricted to it is a
// quadratic in tau solved in closed form (the S0/S1/S2 form of AdaSplash-2
// appendix C.3).  P is written from the register copy, so HBM sees one read
// and one write per element.  Rows wider than the register capacity stream
// the row three times (max, candidates, output).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.hpp"
#include "launch.hpp"

namespace entmax {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kCandCap = 4096;  // candidate floats kept in LDS per row
constexpr int kMaxIter = 48;

struct RowSums {
    float C, S1, S2, F, F1, mn;
};

// Workgroup all-reduce of the six refinement sums (min for mn); slot
// alternates between calls so one barrier per call suffices.
__device__ __forceinline__ RowSums block_reduce(RowSums s, float (*red)[kWaves][6], int slot) {
    const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
    s.C = wave_sum(s.C);
    s.S1 = wave_sum(s.S1);
    s.S2 = wave_sum(s.S2);
    s.F = wave_sum(s.F);
    s.F1 = wave_sum(s.F1);
    s.mn = wave_min(s.mn);
    if (lane == 0) {
        red[slot][w][0] = s.C;
        red[slot][w][1] = s.S1;
        red[slot][w][2] = s.S2;
        red[slot][w][3] = s.F;
        red[slot][w][4] = s.F1;
        red[slot][w][5] = s.mn;
    }
    __syncthreads();
    RowSums r = {0.f, 0.f, 0.f, 0.f, 0.f, __builtin_inff()};
#pragma unroll
    for (int i = 0; i < kWaves; ++i) {
        r.C += red[slot][i][0];
        r.S1 += red[slot][i][1];
        r.S2 += red[slot][i][2];
        r.F += red[slot][i][3];
        r.F1 += red[slot][i][4];
        r.mn = fminf(r.mn, red[slot][i][5]);
    }
    return r;
}

__device__ __forceinline__ float block_max(float v, float* buf) {
    const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
    v = wave_max(v);
    if (lane == 0) buf[w] = v;
    __syncthreads();
    float r = buf[0];
#pragma unroll
    for (int i = 1; i < kWaves; ++i) r = fmaxf(r, buf[i]);
    return r;
}

__device__ __forceinline__ void accumulate(RowSums& s, float x, float t, float m) {
    if (x > t) {
        const float y = x - m;
        const float g = 0.5f * (x - t);
        s.C += 1.0f;
        s.S1 += y;
        s.S2 += y * y;
        s.F += g * g;
        s.F1 += g;
        s.mn = fminf(s.mn, x);
    }
}

// Halley-bisection with exact finish.  `visit(t, sums)` adds this thread's
// contribution at threshold t.  Every thread returns the same tau.
template <class Visit>
__device__ float refine_tau(float m, float total, Visit visit, float (*red)[kWaves][6]) {
    float lo = m - 2.0f;
    float hi = m - 2.0f / sqrtf(total);
    float t = lo;
    for (int it = 0; it < kMaxIter; ++it) {
        RowSums s = {0.f, 0.f, 0.f, 0.f, 0.f, __builtin_inff()};
        visit(t, s);
        s = block_reduce(s, red, it & 1);
        const float f = s.F - 1.0f;
        if (f >= 0.0f) {
            // {x > t} contains the support; if the closed-form root of that
            // set lies below its smallest member, the set is the support.
            const float ts = support_root(m, s.C, s.S1, s.S2);
            if (ts < s.mn) return fmaxf(ts, t);
            lo = t;
        } else {
            hi = t;
        }
        if (hi - lo <= 4e-7f * fmaxf(1.0f, fabsf(t))) break;
        t = halley_or_bisect(t, s.F, s.F1, s.C, lo, hi);
    }
    return 0.5f * (lo + hi);
}

__device__ __forceinline__ float prob(float x, float tau) {
    const float g = fmaxf(0.5f * (x - tau), 0.0f);
    return g * g;
}

// Register-resident row: VPT values per thread.  VEC: float4 accesses
// (ld % 4 == 0 and 16-byte aligned S / P); otherwise scalar accesses.
template <int VPT, bool VEC>
__global__ __launch_bounds__(kThreads) void tau_rows_reg(const float* __restrict__ S,
                                                        float* __restrict__ P,
                                                        float* __restrict__ tau_out,
                                                        int cols, int64_t ld) {
    __shared__ float cand[kCandCap];
    __shared__ float red[2][kWaves][6];
    __shared__ float mbuf[kWaves];
    __shared__ int wcnt[kWaves];

    const int t = threadIdx.x, lane = t & (kWave - 1), w = t / kWave;
    const int64_t row = blockIdx.x;
    const float* src = S + row * ld;
    float v[VPT];

    if constexpr (VEC) {
#pragma unroll
        for (int k = 0; k < VPT / 4; ++k) {
            const int pos = (t + kThreads * k) * 4;
            if (pos + 3 < cols) {
                const f32x4 q = *reinterpret_cast<const f32x4*>(src + pos);
                v[4 * k + 0] = q[0];
                v[4 * k + 1] = q[1];
                v[4 * k + 2] = q[2];
                v[4 * k + 3] = q[3];
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) v[4 * k + e] = (pos + e < cols) ? src[pos + e] : neg_inf();
            }
        }
    } else {
#pragma unroll
        for (int k = 0; k < VPT; ++k) {
            const int pos = t + kThreads * k;
            v[k] = (pos < cols) ? src[pos] : neg_inf();
        }
    }

    float mx = neg_inf();
#pragma unroll
    for (int k = 0; k < VPT; ++k) mx = fmaxf(mx, v[k]);
    const float m = block_max(mx, mbuf);

    float tau;
    if (m == neg_inf()) {
        tau = neg_inf();  // no active entry: P = 0
    } else {
        const float lo0 = m - 2.0f;
        uint32_t cnt = 0;
#pragma unroll
        for (int k = 0; k < VPT; ++k) cnt += __popcll(__ballot(v[k] > lo0));
        if (lane == 0) wcnt[w] = (int)cnt;
        __syncthreads();
        int base = 0, total = 0;
#pragma unroll
        for (int i = 0; i < kWaves; ++i) {
            base += (i < w) ? wcnt[i] : 0;
            total += wcnt[i];
        }
        if (total <= kCandCap) {
            int off = base;
#pragma unroll
            for (int k = 0; k < VPT; ++k) {
                const bool c = v[k] > lo0;
                const uint64_t b = __ballot(c);
                if (c) cand[off + lanes_below(b)] = v[k];
                off += __popcll(b);
            }
            __syncthreads();
            tau = refine_tau(
                m, (float)total,
                [&](float tt, RowSums& s) {
                    for (int i = t; i < total; i += kThreads) accumulate(s, cand[i], tt, m);
                },
                red);
        } else {
            tau = refine_tau(
                m, (float)total,
                [&](float tt, RowSums& s) {
#pragma unroll
                    for (int k = 0; k < VPT; ++k) accumulate(s, v[k], tt, m);
                },
                red);
        }
    }

    if (t == 0) tau_out[row] = tau;
    if (P == nullptr) return;
    float* dst = P + row * ld;
    if constexpr (VEC) {
#pragma unroll
        for (int k = 0; k < VPT / 4; ++k) {
            const int pos = (t + kThreads * k) * 4;
            if (pos + 3 < cols) {
                f32x4 q;
                q[0] = prob(v[4 * k + 0], tau);
                q[1] = prob(v[4 * k + 1], tau);
                q[2] = prob(v[4 * k + 2], tau);
                q[3] = prob(v[4 * k + 3], tau);
                __builtin_nontemporal_store(q, reinterpret_cast<f32x4*>(dst + pos));
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (pos + e < cols) dst[pos + e] = prob(v[4 * k + e], tau);
            }
        }
    } else {
#pragma unroll
        for (int k = 0; k < VPT; ++k) {
            const int pos = t + kThreads * k;
            if (pos < cols) dst[pos] = prob(v[k], tau);
        }
    }
}

// Any width: the row is streamed from global memory (L2-resident after the
// first pass for moderate widths).
__global__ __launch_bounds__(kThreads) void tau_rows_stream(const float* __restrict__ S,
                                                           float* __restrict__ P,
                                                           float* __restrict__ tau_out,
                                                           int64_t cols, int64_t ld) {
    __shared__ float cand[kCandCap];
    __shared__ float red[2][kWaves][6];
    __shared__ float mbuf[kWaves];
    __shared__ int wcnt[kWaves];

    const int t = threadIdx.x, lane = t & (kWave - 1), w = t / kWave;
    const int64_t row = blockIdx.x;
    const float* src = S + row * ld;

    float mx = neg_inf();
    for (int64_t pos = t; pos < cols; pos += kThreads) mx = fmaxf(mx, src[pos]);
    const float m = block_max(mx, mbuf);

    float tau;
    if (m == neg_inf()) {
        tau = neg_inf();
    } else {
        const float lo0 = m - 2.0f;
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
            filled += tot;
            __syncthreads();
        }
        if (filled <= kCandCap) {
            tau = refine_tau(
                m, (float)filled,
                [&](float tt, RowSums& s) {
                    for (int i = t; i < filled; i += kThreads) accumulate(s, cand[i], tt, m);
                },
                red);
        } else {
            tau = refine_tau(
                m, (float)filled,
                [&](float tt, RowSums& s) {
                    for (int64_t pos = t; pos < cols; pos += kThreads) accumulate(s, src[pos], tt, m);
                },
                red);
        }
    }
    if (t == 0) tau_out[row] = tau;
    if (P == nullptr) return;
    float* dst = P + row * ld;
    for (int64_t pos = t; pos < cols; pos += kThreads) dst[pos] = prob(src[pos], tau);
}

template <int VPT, bool VEC>
hipError_t launch_reg(const float* S, float* P, float* tau, int64_t rows, int64_t cols,
                      int64_t ld, hipStream_t stream) {
    hipLaunchKernelGGL((tau_rows_reg<VPT, VEC>), dim3((unsigned)rows), dim3(kThreads), 0,
                       stream, S, P, tau, (int)cols, ld);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_tau_rows(const float* S, float* P, float* tau, int64_t rows, int64_t cols,
                           int64_t ld, hipStream_t stream) {
    const bool vec = (ld % 4 == 0) && ((uintptr_t)S % 16 == 0) &&
                     (P == nullptr || (uintptr_t)P % 16 == 0);
    if (vec) {
        if (cols <= 1 * 4 * kThreads) return launch_reg<4, true>(S, P, tau, rows, cols, ld, stream);
        if (cols <= 2 * 4 * kThreads) return launch_reg<8, true>(S, P, tau, rows, cols, ld, stream);
        if (cols <= 4 * 4 * kThreads) return launch_reg<16, true>(S, P, tau, rows, cols, ld, stream);
        if (cols <= 8 * 4 * kThreads) return launch_reg<32, true>(S, P, tau, rows, cols, ld, stream);
    } else {
        if (cols <= 4 * kThreads) return launch_reg<4, false>(S, P, tau, rows, cols, ld, stream);
        if (cols <= 8 * kThreads) return launch_reg<8, false>(S, P, tau, rows, cols, ld, stream);
        if (cols <= 16 * kThreads) return launch_reg<16, false>(S, P, tau, rows, cols, ld, stream);
        if (cols <= 32 * kThreads) return launch_reg<32, false>(S, P, tau, rows, cols, ld, stream);
    }
    hipLaunchKernelGGL(tau_rows_stream, dim3((unsigned)rows), dim3(kThreads), 0, stream, S, P,
                       tau, cols, ld);
    return hipGetLastError();
}

}  // namespace entmax
