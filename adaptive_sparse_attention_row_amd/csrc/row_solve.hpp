// row_solve.hpp -- threshold solves over a score row held by one wave or by
// a 256-thread workgroup (in registers, compacted into LDS, or streamed from
// memory): shared by the row kernel and the decode step.
//
// alpha = 1.5: Halley-bisection (the hybrid solver of "AdaSplash: Adaptive
// Sparse Flash Attention", summary, Approach) on the bracket
// [m - 2, m - 2/sqrt(n)] of "AdaSplash-2: Faster Differentiable Sparse
// Attention" sec. 2.4 in score units, with an exact finish: once {s > t} is
// the support, the normaliser over it is a quadratic in tau (the S0/S1/S2
// form of AdaSplash-2 appendix C.3).  Other alpha in (1, 2]: Newton steps
// from below with a bisection guard (newton_or_bisect).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.hpp"

namespace entmax {
namespace rows {

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
__device__ float refine_tau(float m, float total, Visit visit, float (*red)[kWaves][6],
                           float lo_in = -__builtin_inff(), float hi_in = __builtin_inff()) {
    // the bracket [m - 2, m - 2/sqrt(n)], narrowed to [lo_in, hi_in] when given
    float lo = fmaxf(m - 2.0f, lo_in);
    float hi = fminf(m - 2.0f / sqrtf(total), hi_in);
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

// prob() with h = -tau/2 precomputed: fma(x, 1/2, h) rounds 0.5x - 0.5tau,
// and halving is exact, so this equals 0.5 * (x - tau) bit for bit.
__device__ __forceinline__ float prob_h(float x, float h) {
    const float g = fmaxf(__builtin_fmaf(x, 0.5f, h), 0.0f);
    return g * g;
}

// General alpha: this thread's F = sum p and F1 = sum p/u at threshold t.
__device__ __forceinline__ void accumulate_gen(RowSums& s, float x, float t, const AlphaMap& a) {
    const float u = a.am1 * (x - t);
    if (u > 0.0f) {
        const float q = a.pw1(u);  // p / u
        s.F = fmaf(q, u, s.F);
        s.F1 += q;
    }
}

// Workgroup form of wave_tau_gen for the streaming kernel.
template <class Visit>
__device__ float refine_tau_gen(float m, float total, const AlphaMap& a, Visit visit,
                                float (*red)[kWaves][6], float lo_in = -__builtin_inff(),
                                float hi_in = __builtin_inff()) {
    float lo = fmaxf(m - a.e, lo_in);
    float hi = fminf(a.hi(m, total), hi_in);
    float t = lo;
    for (int it = 0; it < kMaxIter; ++it) {
        RowSums s = {0.f, 0.f, 0.f, 0.f, 0.f, __builtin_inff()};
        visit(t, s);
        s = block_reduce(s, red, it & 1);
        bool done;
        const float tn = newton_or_bisect(t, s.F, s.F1, lo, hi, &done, a);
        if (done) return tn;
        if (hi - lo <= 4e-7f * fmaxf(1.0f, fabsf(t))) break;
        t = tn;
    }
    return 0.5f * (lo + hi);
}

// Histogram initialisation ("AdaSplash-2: Faster Differentiable Sparse
// Attention" sec. 3.1, appendix C.3), in the pages' z-units:
//   z = (alpha - 1)(s - m) + 1  (z = 1 at the maximum; only z >= 0 can carry
//   weight), bin k = min(floor(B z), B - 1) (left edges).
// Replacing every z by its bin's left edge k/B can only lower the normaliser,
// so the histogram threshold tau_h (the root of sum_k H_k [k/B - tau]_+^e = 1)
// satisfies tau* - 1/B < tau_h <= tau* (Proposition 3.1): in score units
// tau lies in [tau_h, tau_h + 1/(B (alpha - 1))].
constexpr int kHistBins = 64;

__device__ __forceinline__ int hist_bin(float x, float m, float am1) {
    const float z = __builtin_fmaf(am1, x - m, 1.0f);
    int k = (int)floorf(z * (float)kHistBins);
    k = k < kHistBins - 1 ? k : kHistBins - 1;
    return k > 0 ? k : 0;
}

// tau_h from the bin counts (one count per lane, lane k = bin k of a 64-lane
// wave): bisection on the histogram objective over [(B-1)/B - 1, (B-1)/B]
// (the top bin, which holds the maximum, gives f_h >= 0 at the lower end),
// every lane taking part.  Returned in score units.
__device__ __forceinline__ float hist_tau(int count, float m, const AlphaMap& a) {
    static_assert(kHistBins == kWave, "one bin per lane");
    const float edge = (float)lane_id() / (float)kHistBins;
    const float c = (float)count;
    float lo = (float)(kHistBins - 1) / kHistBins - 1.0f, hi = (float)(kHistBins - 1) / kHistBins;
    for (int it = 0; it < 40; ++it) {
        const float mid = 0.5f * (lo + hi);
        if (!(mid > lo && mid < hi)) break;
        const float u = edge - mid;
        float f = (u > 0.0f && c > 0.0f) ? c * (a.lin ? u : exp2f(a.e * log2f(u))) : 0.0f;
        // wave sum by butterfly (all lanes end with the total)
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) f += __shfl_xor(f, o, kWave);
        if (f >= 1.0f) lo = mid;
        else hi = mid;
    }
    return m + (lo - 1.0f) * a.e;
}

// DPP sum / min over the 64 lanes of a wave, result in every lane.  Lanes
// with no source in a step read the identity (0 or +inf).
__device__ __forceinline__ float wave_sum_dpp(float x) {
#define ENTMAX_DPP_STEP(op, idv, ctrl, rmask)                                                  \
    x = op(x, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(                           \
                  __builtin_bit_cast(int, idv), __builtin_bit_cast(int, x), ctrl, rmask, 0xf, \
                  false)))
#define ENTMAX_ADD(a, b) ((a) + (b))
    ENTMAX_DPP_STEP(ENTMAX_ADD, 0.0f, 0x111, 0xf);
    ENTMAX_DPP_STEP(ENTMAX_ADD, 0.0f, 0x112, 0xf);
    ENTMAX_DPP_STEP(ENTMAX_ADD, 0.0f, 0x114, 0xf);
    ENTMAX_DPP_STEP(ENTMAX_ADD, 0.0f, 0x118, 0xf);
    ENTMAX_DPP_STEP(ENTMAX_ADD, 0.0f, 0x142, 0xa);
    ENTMAX_DPP_STEP(ENTMAX_ADD, 0.0f, 0x143, 0xc);
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 63));
}
__device__ __forceinline__ float wave_min_dpp(float x) {
    ENTMAX_DPP_STEP(fminf, __builtin_inff(), 0x111, 0xf);
    ENTMAX_DPP_STEP(fminf, __builtin_inff(), 0x112, 0xf);
    ENTMAX_DPP_STEP(fminf, __builtin_inff(), 0x114, 0xf);
    ENTMAX_DPP_STEP(fminf, __builtin_inff(), 0x118, 0xf);
    ENTMAX_DPP_STEP(fminf, __builtin_inff(), 0x142, 0xa);
    ENTMAX_DPP_STEP(fminf, __builtin_inff(), 0x143, 0xc);
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 63));
}
__device__ __forceinline__ float wave_max_dpp(float x) {
    ENTMAX_DPP_STEP(fmaxf, neg_inf(), 0x111, 0xf);
    ENTMAX_DPP_STEP(fmaxf, neg_inf(), 0x112, 0xf);
    ENTMAX_DPP_STEP(fmaxf, neg_inf(), 0x114, 0xf);
    ENTMAX_DPP_STEP(fmaxf, neg_inf(), 0x118, 0xf);
    ENTMAX_DPP_STEP(fmaxf, neg_inf(), 0x142, 0xa);
    ENTMAX_DPP_STEP(fmaxf, neg_inf(), 0x143, 0xc);
#undef ENTMAX_ADD
#undef ENTMAX_DPP_STEP
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 63));
}

// Exclusive prefix sum of a count over the 64 lanes of a wave (DPP row
// shifts build the inclusive scan inside each row of 16 lanes, two row
// broadcasts carry it across rows); *total receives the wave's sum.
__device__ __forceinline__ int wave_excl_scan(int x, int* total) {
    int y = x;
#define ENTMAX_SCAN_STEP(ctrl, rmask) y += __builtin_amdgcn_update_dpp(0, y, ctrl, rmask, 0xf, false)
    ENTMAX_SCAN_STEP(0x111, 0xf);
    ENTMAX_SCAN_STEP(0x112, 0xf);
    ENTMAX_SCAN_STEP(0x114, 0xf);
    ENTMAX_SCAN_STEP(0x118, 0xf);
    ENTMAX_SCAN_STEP(0x142, 0xa);
    ENTMAX_SCAN_STEP(0x143, 0xc);
#undef ENTMAX_SCAN_STEP
    *total = __builtin_amdgcn_readlane(y, 63);
    return y - x;
}

// A lower bound on the 1.5-entmax threshold of a row from one of its values
// per lane (a subset, e.g. each lane's maximum; -inf for none): Newton steps
// from t = m - 2 on the subset's f(t) = sum [(x - t)/2]_+^2 - 1.  f is convex
// and decreasing and f(m - 2) >= 0 (the maximum alone contributes 1), so
// every step stays at or below the subset's threshold, which is at most the
// row's (adding scores only raises a threshold).  The steps stop once f is
// below 1e-2 (the bound is then within about 1e-2 of the subset's
// threshold); the result is lowered by a relative 1e-5, more than the
// rounding of the fp32 sums can move a step (|dF| / F1 <= 64 ulp, since
// F / F1 <= max g <= 1 and F1 >= 1 below the root).
__device__ __forceinline__ float wave_newton_lower(float x, float m) {
    float t = m - 2.0f;
#pragma unroll 1
    for (int it = 0; it < 8; ++it) {
        const float g = fmaxf(0.5f * (x - t), 0.0f);
        const float f = wave_sum_dpp(g * g) - 1.0f;
        const float F1 = wave_sum_dpp(g);
        if (f <= 1e-2f) break;
        t += f / F1;
    }
    return t - 1e-5f * fmaxf(1.0f, fabsf(t));
}

// Threshold of a set held by one wave: `each(t, sums)` adds this lane's part
// of the sums over {x > t}.  Halley-bisection in the bracket [lo, m - 2/sqrt(n)]
// (lo a lower bound on tau, no smaller than m - 2; n >= the support size)
// with the exact finish of refine_tau; all sums are wave reductions.  Every
// lane returns the same tau.
template <class Each>
__device__ __forceinline__ float wave_tau(float m, float n, float lo, Each each) {
    float hi = m - 2.0f / sqrtf(n);
    float t = lo;
    for (int it = 0; it < kMaxIter; ++it) {
        RowSums s = {0.f, 0.f, 0.f, 0.f, 0.f, __builtin_inff()};
        each(t, s);
        s.C = wave_sum_dpp(s.C);
        s.S1 = wave_sum_dpp(s.S1);
        s.S2 = wave_sum_dpp(s.S2);
        s.F = wave_sum_dpp(s.F);
        s.F1 = wave_sum_dpp(s.F1);
        s.mn = wave_min_dpp(s.mn);
        if (s.F - 1.0f >= 0.0f) {
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

// General-alpha threshold of a set held by one wave (Newton from below, see
// newton_or_bisect) in [lo, hi(m, n)].  Every lane returns the same tau;
// *lo_out receives the final lower bracket end (a point with f >= 0, so a
// lower bound on tau up to the rounding of the sums).
template <class Each>
__device__ __forceinline__ float wave_tau_gen(float m, float n, float lo, const AlphaMap& a, Each each,
                                              float* lo_out) {
    float hi = a.hi(m, n);
    float t = lo;
    float tau = 0.5f * (lo + hi);
    for (int it = 0; it < kMaxIter; ++it) {
        RowSums s = {0.f, 0.f, 0.f, 0.f, 0.f, __builtin_inff()};
        each(t, s);
        s.F = wave_sum_dpp(s.F);
        s.F1 = wave_sum_dpp(s.F1);
        bool done;
        const float tn = newton_or_bisect(t, s.F, s.F1, lo, hi, &done, a);
        if (done) {
            tau = tn;
            break;
        }
        if (hi - lo <= 4e-7f * fmaxf(1.0f, fabsf(t))) {
            tau = 0.5f * (lo + hi);
            break;
        }
        t = tn;
        tau = 0.5f * (lo + hi);
    }
    if (lo_out) *lo_out = lo;
    return tau;
}

}  // namespace rows
}  // namespace entmax
