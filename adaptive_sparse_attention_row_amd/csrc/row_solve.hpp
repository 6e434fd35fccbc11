// row_solve.hpp -- threshold solves over one score row held by a 256-thread
// workgroup (the row streamed from memory or compacted into LDS): shared by
// the wide-row path of the row kernel and the decode step.
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
        const float p = a.pw(u);
        s.F += p;
        s.F1 += p / u;
    }
}

// Workgroup form of wave_tau_gen for the streaming kernel.
template <class Visit>
__device__ float refine_tau_gen(float m, float total, const AlphaMap& a, Visit visit,
                                float (*red)[kWaves][6]) {
    float lo = m - a.e;
    float hi = a.hi(m, total);
    float t = lo;
    for (int it = 0; it < kMaxIter; ++it) {
        RowSums s = {0.f, 0.f, 0.f, 0.f, 0.f, __builtin_inff()};
        visit(t, s);
        s = block_reduce(s, red, it & 1);
        bool done;
        const float tn = newton_or_bisect(t, s.F, s.F1, lo, hi, &done);
        if (done) return tn;
        if (hi - lo <= 4e-7f * fmaxf(1.0f, fabsf(t))) break;
        t = tn;
    }
    return 0.5f * (lo + hi);
}

}  // namespace rows
}  // namespace entmax
