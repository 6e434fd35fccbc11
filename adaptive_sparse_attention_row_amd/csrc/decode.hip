// decode.hip -- one decode step of alpha-entmax attention: the newest query
// of every (batch, head), at position L - 1, against its KV cache.
//
// "AdaSplash-2: Faster Differentiable Sparse Attention" names inference as
// further work; the GPT-2 model card generates with a causal window of W
// recent keys plus the sink key 0 (Mathematical Formulation item 1).  The
// step computes exactly the last row of the forward:
//   s_j = scale q . K_j over the active keys, tau from sum_j p_j = 1,
//   o = sum_j p_j V_j.
// Only the support carries weight, so only the support's rows of V are read:
// the forward's block traversal (AdaSplash-2 sec. 3.3 phase 4) taken down to
// single keys.  HBM traffic is the K cache of the active keys plus a few
// dozen V rows, about half of what a dense decode reads.
//
// dec_scores  grid (active keys / 256, B*H): each wave dots 64 keys with the
//             query.  A K row is LPK = d * esize / 16 chunks of 16 bytes; one
//             load instruction covers 64 / LPK whole rows (each lane a chunk
//             of one row, so a wave reads 1 KiB contiguous), and after LPK
//             instructions the LPK lanes of a row group hold LPK partial sums
//             of LPK keys: a reduce-scatter of LPK - 1 lane exchanges leaves
//             lane c with the full dot of key c.  Scores go to the workspace.
// dec_solve   one 256-thread workgroup per (batch, head): each wave scans a
//             quarter of the score row (its lane maxima and their threshold,
//             a lower bound on tau; then the scores above the largest of the
//             four bounds, with their positions, into its own LDS list); tau
//             by the row solves of row_solve.hpp over the four lists (at
//             alpha = 1.5 each wave solves on all of them with wave
//             reductions, starting from the bound); then o
//             from the support's V rows only (the threads split the head
//             dimension, groups of them split the support, and the groups
//             are summed through LDS).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "device_common.hpp"
#include "launch.hpp"
#include "row_solve.hpp"

namespace entmax {
namespace dec {
namespace {

using namespace rows;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

struct DecParams {
    const void* q;  // [BH][d]
    const void* k;  // [BH][Lcap][d]
    const void* v;  // [BH][Lcap][d]
    float* o;       // [BH][d]
    float* tau;     // [BH]
    float* s;       // workspace [BH][nact]: scores of the active keys
    int BH, L, Lcap, nact, j0;  // active keys: 0 (when j0 > 0), then j0 .. L - 1
    float scale;
    AlphaMap am;
    int gen;  // alpha != 1.5
};

// Position in the active-key list -> key index.
__device__ __forceinline__ int key_of(int pos, int j0) {
    if (j0 == 0) return pos;
    return pos == 0 ? 0 : j0 + pos - 1;
}

template <typename T>
__device__ __forceinline__ void unpack(const u32x4& c, float (&x)[16 / sizeof(T)]) {
    if constexpr (sizeof(T) == 2) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[2 * i] = __builtin_bit_cast(float, c[i] << 16);
            x[2 * i + 1] = __builtin_bit_cast(float, c[i] & 0xffff0000u);
        }
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            // (a vector element taken straight into __builtin_bit_cast came out
            // as element 0 for every i with this compiler: copy it first)
            const uint32_t wv = c[i];
            x[i] = __builtin_bit_cast(float, wv);
        }
    }
}

// The value of lane l ^ hh (hh a power of two below 32), without LDS where
// a DPP pattern has it: a rotation by 8 within each row of 16 lanes for 8, the
// quad permutations for 2 and 1; ds_swizzle's xor mode otherwise.
__device__ __forceinline__ float xor_lanes(float x, int hh) {
    const int v = __builtin_bit_cast(int, x);
    if (hh == 8) return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(v, 0x128, 0xf, 0xf, false));
    if (hh == 2) return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(v, 0x4e, 0xf, 0xf, false));
    if (hh == 1) return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(v, 0xb1, 0xf, 0xf, false));
    if (hh == 4) return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(v, 0x1f | (4 << 10)));
    if (hh == 16) return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(v, 0x1f | (16 << 10)));
    return __shfl_xor(x, hh, kWave);
}

template <typename T, int D>
__global__ __launch_bounds__(256) void dec_scores(DecParams p) {
    constexpr int kEpc = 16 / sizeof(T);            // elements per 16-byte chunk
    constexpr int kLpk = D * (int)sizeof(T) / 16;    // lanes (chunks) per key row
    constexpr int kKpi = kWave / kLpk;               // key rows per load instruction
    const int bh = blockIdx.y;
    const int w = wave_id(), l = lane_id();
    const int c = l % kLpk, grp = l / kLpk;
    const int p0 = blockIdx.x * 256 + w * kWave;     // first active position of this wave
    if (p0 >= p.nact) return;

    // this lane's slice of the query
    float qv[kEpc];
    {
        const u32x4 qc = reinterpret_cast<const u32x4*>(reinterpret_cast<const T*>(p.q) + (size_t)bh * D)[c];
        unpack<T>(qc, qv);
    }
    const T* Kh = reinterpret_cast<const T*>(p.k) + (size_t)bh * p.Lcap * D;
    // Every load of the wave is issued before the first product.  (Written
    // as two lambdas over the chunk array: the same steps written inline
    // compiled the reduce-scatter's selects into a select chain over all of
    // part[], 3.4x the instructions and 5 % slower.)
    auto load_all = [&](u32x4 (&kc)[kLpk]) {
#pragma unroll
        for (int i = 0; i < kLpk; ++i) {
            int pos = p0 + i * kKpi + grp;
            pos = pos < p.nact ? pos : p.nact - 1;  // tail lanes repeat the last key; never stored
            const int key = key_of(pos, p.j0);
            kc[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(Kh + (size_t)key * D) + c);
        }
    };
    auto finish = [&](const u32x4 (&kc)[kLpk]) {
        float part[kLpk];
#pragma unroll
        for (int i = 0; i < kLpk; ++i) {
            float kv[kEpc];
            unpack<T>(kc[i], kv);
            float acc = 0.f;
#pragma unroll
            for (int e = 0; e < kEpc; ++e) acc = fmaf(qv[e], kv[e], acc);
            part[i] = acc;
        }
        // reduce-scatter over the kLpk lanes of the row group: after the step
        // with offset hh, lane c keeps the half of its keys selected by bit hh of c
#pragma unroll
        for (int hh = kLpk / 2; hh >= 1; hh >>= 1) {
            const bool up = (c & hh) != 0;
#pragma unroll
            for (int j = 0; j < hh; ++j) {
                const float mine = up ? part[j + hh] : part[j];
                const float other = up ? part[j] : part[j + hh];
                part[j] = mine + xor_lanes(other, hh);
            }
        }
        const int pos = p0 + c * kKpi + grp;  // the key whose dot lane c now holds
        if (pos < p.nact) p.s[(size_t)bh * p.nact + pos] = part[0] * p.scale;
    };
    u32x4 kc[kLpk];
    load_all(kc);
    finish(kc);
}

constexpr int kDecCap = 4096;            // candidates kept in LDS per (batch, head)
constexpr int kWaveCap = kDecCap / kWaves; // ... as four per-wave lists

template <typename T, int D>
__global__ __launch_bounds__(256) void dec_solve(DecParams p) {
    __shared__ float cv[kDecCap];
    __shared__ int cp[kDecCap];
    __shared__ float red[2][kWaves][6];
    __shared__ float mbuf[kWaves], wbnd[kWaves];
    __shared__ int wcnt[kWaves];
    __shared__ float osum[4 * 256];

    const int t = threadIdx.x, lane = t & (kWave - 1), w = wave_id();
    const int bh = blockIdx.x;
    const int n = p.nact;
    const float* srow = p.s + (size_t)bh * n;

    // Each wave scans a quarter of the score row.  Pass 1: the lane maxima,
    // and a lower bound on the threshold of those 64 values (the row kernel's
    // bound: they are a subset of the row, and a threshold only rises as
    // scores are added, so it is a lower bound on tau).  The largest of the
    // four waves' bounds is the row's candidate threshold.  Pass 2: every
    // score above it, with its position, into the wave's own LDS list.  A
    // quarter of up to kNB * kU * kWave scores (rows of up to 16384 keys) is
    // loaded once, all of it in flight together, and pass 2 reads the
    // registers; longer rows are read in steps of kU loads per lane, twice.
    constexpr int kU = 16, kNB = 4;
    const int q0 = (int)(((int64_t)n * w) / kWaves), q1 = (int)(((int64_t)n * (w + 1)) / kWaves);
    auto load16 = [&](int base, float (&x)[kU]) {
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const int i = base + u * kWave + lane;
            x[u] = i < q1 ? srow[i] : neg_inf();
        }
    };
    const bool inreg = (q1 - q0) <= kNB * kU * kWave;  // per wave: quarters differ by at most one
    float xr[kNB][kU];
    float lm = neg_inf();
    if (inreg) {
#pragma unroll
        for (int b = 0; b < kNB; ++b) {
            load16(q0 + b * kU * kWave, xr[b]);
#pragma unroll
            for (int u = 0; u < kU; ++u) lm = fmaxf(lm, xr[b][u]);
        }
    } else {
        for (int base = q0; base < q1; base += kU * kWave) {
            float x[kU];
            load16(base, x);
#pragma unroll
            for (int u = 0; u < kU; ++u) lm = fmaxf(lm, x[u]);
        }
    }
    const float wm = wave_max_dpp(lm);
    float wlo = neg_inf();
    if (wm > neg_inf()) {
        if (p.gen) {
            const float n1 = wave_sum_dpp(lm > neg_inf() ? 1.0f : 0.0f);
            wave_tau_gen(wm, n1, wm - p.am.e, p.am, [&](float tt, RowSums& s) { accumulate_gen(s, lm, tt, p.am); },
                         &wlo);
        } else {
            wlo = wave_newton_lower(lm, wm);
        }
    }
    if (lane == 0) {
        mbuf[w] = wm;
        wbnd[w] = wlo;
    }
    __syncthreads();
    float m = mbuf[0], bound = wbnd[0];
#pragma unroll
    for (int k = 1; k < kWaves; ++k) {
        m = fmaxf(m, mbuf[k]);
        bound = fmaxf(bound, wbnd[k]);
    }
    float* wv = cv + w * kWaveCap;
    int* wp = cp + w * kWaveCap;
    int cnt = 0;
    // append the scores of x above the bound (positions base + u * kWave + lane)
    auto compact = [&](int base, const float (&x)[kU]) {
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const bool is_c = x[u] > bound;
            const uint64_t b = __ballot(is_c);
            if (b == 0) continue;
            const int slot = cnt + lanes_below(b);
            if (is_c && slot < kWaveCap) {
                wv[slot] = x[u];
                wp[slot] = base + u * kWave + lane;
            }
            cnt += __popcll(b);
        }
    };
    if (inreg) {
#pragma unroll
        for (int b = 0; b < kNB; ++b) compact(q0 + b * kU * kWave, xr[b]);
    } else {
        for (int base = q0; base < q1; base += kU * kWave) {
            float x[kU];
            load16(base, x);
            compact(base, x);
        }
    }
    if (lane == 0) wcnt[w] = cnt;
    __syncthreads();
    int filled = 0;
    bool fits = true;
#pragma unroll
    for (int k = 0; k < kWaves; ++k) {
        filled += wcnt[k];
        fits = fits && wcnt[k] <= kWaveCap;
    }
    // visit the candidates of the four lists (thread t: entries t, t + 256, ...)
    auto each_cand = [&](auto f) {
#pragma unroll
        for (int k = 0; k < kWaves; ++k)
            for (int i = t; i < wcnt[k]; i += 256) f(cv[k * kWaveCap + i], cp[k * kWaveCap + i]);
    };

    float tau;
    if (p.gen) {
        tau = fits ? refine_tau_gen(m, (float)filled, p.am, [&](float tt, RowSums& s) {
            each_cand([&](float x, int) { accumulate_gen(s, x, tt, p.am); });
        }, red)
                   : refine_tau_gen(m, (float)filled, p.am, [&](float tt, RowSums& s) {
            for (int i = t; i < n; i += 256) accumulate_gen(s, srow[i], tt, p.am);
        }, red);
    } else if (fits) {
        // every wave solves on all four lists with wave reductions only (the
        // same sums in the same order, so the same tau), from the bound:
        // tau >= m - 2 (the maximum alone has weight 1) and tau >= bound
        tau = wave_tau(m, (float)filled, fmaxf(bound, m - 2.0f), [&](float tt, RowSums& s) {
#pragma unroll
            for (int k = 0; k < kWaves; ++k)
                for (int i = lane; i < wcnt[k]; i += kWave) accumulate(s, cv[k * kWaveCap + i], tt, m);
        });
    } else {
        tau = refine_tau(m, (float)filled, [&](float tt, RowSums& s) {
            for (int i = t; i < n; i += 256) accumulate(s, srow[i], tt, m);
        }, red);
    }

    // o = sum over the support of p_j V_j.  Each wave first compacts the
    // support of its own list in place (weight, key), in list order, so the
    // sum below runs in a fixed order.  Then thread t takes 4 consecutive
    // dimensions of every kG-th support entry (kG = 256 / (D / 4) groups, so
    // all of a short support's V rows are in flight at once), and the groups
    // are summed through LDS.
    auto weight = [&](float x) -> float {
        if (p.gen) return p.am.p(x, tau);
        const float gg = fmaxf(0.5f * (x - tau), 0.0f);
        return gg * gg;
    };
    const T* Vh = reinterpret_cast<const T*>(p.v) + (size_t)bh * p.Lcap * D;
    constexpr int kQ = D / 4;        // threads per V row (4 dimensions each)
    constexpr int kG = 256 / kQ;     // support entries in flight
    const int d4 = (t % kQ) * 4, g = t / kQ;
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    auto add_row = [&](float wgt, int key) {
        const T* row = Vh + (size_t)key * D + d4;
        if constexpr (sizeof(T) == 2) {
            const u32x2 v2 = *reinterpret_cast<const u32x2*>(row);
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const uint32_t wv2 = v2[e];
                acc[2 * e] = fmaf(wgt, __builtin_bit_cast(float, wv2 << 16), acc[2 * e]);
                acc[2 * e + 1] = fmaf(wgt, __builtin_bit_cast(float, wv2 & 0xffff0000u), acc[2 * e + 1]);
            }
        } else {
            const f32x4 v4 = *reinterpret_cast<const f32x4*>(row);
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[e] = fmaf(wgt, v4[e], acc[e]);
        }
    };
    if (fits) {
        __syncthreads();  // every wave's solve has read all four lists
        const int mine = wcnt[w] < kWaveCap ? wcnt[w] : kWaveCap;
        int ns = 0;
        for (int i0 = 0; i0 < mine; i0 += kWave) {
            const int i = i0 + lane;
            const float x = i < mine ? wv[i] : neg_inf();
            const int pos = i < mine ? wp[i] : 0;
            const bool on = x > tau;
            const uint64_t b = __ballot(on);
            if (on) {
                const int slot = ns + lanes_below(b);
                wv[slot] = weight(x);
                wp[slot] = key_of(pos, p.j0);
            }
            ns += __popcll(b);
        }
        __syncthreads();  // every wave's reads of its list are done before wcnt changes
        if (lane == 0) wcnt[w] = ns;
        __syncthreads();
#pragma unroll
        for (int k = 0; k < kWaves; ++k) {
#pragma unroll 4
            for (int i = g; i < wcnt[k]; i += kG) add_row(cv[k * kWaveCap + i], cp[k * kWaveCap + i]);
        }
    } else {
        for (int i = g; i < n; i += kG) {
            const float x = srow[i];
            if (x > tau) add_row(weight(x), key_of(i, p.j0));
        }
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) osum[g * D + d4 + e] = acc[e];
    __syncthreads();
    if (t < D) {
        float o = 0.f;
#pragma unroll
        for (int k = 0; k < kG; ++k) o += osum[k * D + t];
        p.o[(size_t)bh * D + t] = o;
    }
    if (t == 0) p.tau[bh] = tau;
}

template <typename T, int D>
hipError_t launch_typed(const DecParams& dp, hipStream_t stream) {
    const dim3 g1((unsigned)((dp.nact + 255) / 256), (unsigned)dp.BH);
    hipLaunchKernelGGL((dec_scores<T, D>), g1, dim3(256), 0, stream, dp);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((dec_solve<T, D>), dim3((unsigned)dp.BH), dim3(256), 0, stream, dp);
    return hipGetLastError();
}

}  // namespace
}  // namespace dec

// Active keys of the query at position L - 1: all of [0, L) unless the
// window mode drops the keys more than W behind (the sink key 0 stays).
static void decode_active(int L, int mask, int window, int* j0, int* nact) {
    int s = 0;
    if (mask == 2) {
        const long long lo = (long long)L - 1 - window;
        s = lo > 0 ? (int)lo : 0;
    }
    *j0 = s;
    *nact = (L - s) + (s > 0 ? 1 : 0);
}

size_t attn_decode_workspace_bytes(int B, int H, int L, int mask, int window) {
    int j0, nact;
    decode_active(L, mask, window, &j0, &nact);
    return (size_t)B * H * nact * sizeof(float);
}

hipError_t launch_attn_decode(const AttnArgs& a, int Lcap, hipStream_t stream) {
    using namespace dec;
    DecParams dp;
    dp.q = a.q; dp.k = a.k; dp.v = a.v; dp.o = a.o; dp.tau = a.tau;
    dp.s = reinterpret_cast<float*>(a.workspace);
    dp.BH = a.B * a.H; dp.L = a.L; dp.Lcap = Lcap;
    decode_active(a.L, a.mask, a.window, &dp.j0, &dp.nact);
    dp.scale = a.scale;
    dp.am = make_alpha_map(a.alpha);
    dp.gen = a.alpha != 1.5f ? 1 : 0;
    if (a.dtype == 1) {
        if (a.d == 64) return launch_typed<__bf16, 64>(dp, stream);
        return launch_typed<__bf16, 128>(dp, stream);
    }
    if (a.d == 64) return launch_typed<float, 64>(dp, stream);
    return launch_typed<float, 128>(dp, stream);
}

// ------------------------------------------------ allocation-free decode
// The per-key scores of entmax_attn_decode_noalloc live in this file-scope
// array instead of a caller workspace: every device the library runs on
// holds its own copy, at its own address, until the process ends.  In host
// code `scratch` names a host-side stand-in, so its device address is looked
// up once per device (hipGetSymbolAddress with that device current) and only
// that address is ever handed to a kernel.
__device__ __align__(256) unsigned char scratch[kDecodeScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_addr[kMaxDevices] = {};
}  // namespace

hipError_t decode_scratch_address(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_addr[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_scratch_addr[dev] = p;
    }
    *out = g_scratch_addr[dev];
    return hipSuccess;
}

}  // namespace entmax
