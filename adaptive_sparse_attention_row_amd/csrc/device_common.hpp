// device_common.hpp -- small gfx950 device helpers shared by the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace entmax {

constexpr int kWave = 64;

typedef float f32x4 __attribute__((ext_vector_type(4)));

// Butterfly all-reduce across the 64 lanes of a wavefront.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
    return v;
}

__device__ __forceinline__ float wave_min(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fminf(v, __shfl_xor(v, o, kWave));
    return v;
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Index of this wave in its workgroup, as a scalar (it is the same for every
// lane, and code that depends only on it then stays on the scalar unit).
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x / kWave); }

// Number of set bits of `mask` in lanes below this one.
__device__ __forceinline__ int lanes_below(uint64_t mask) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                     __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

__device__ __forceinline__ float neg_inf() { return -__builtin_inff(); }

// Lane pairs (l, l ^ 32) without LDS: v_permlane32_swap exchanges the upper
// half of its first operand with the lower half of its second, so with x in
// both, the two results hold the x of lanes l & 31 and (l & 31) + 32, in
// every lane l.  Combining them in that order gives both lanes of a pair the
// same bits.
__device__ __forceinline__ void pair_halves(uint32_t x, uint32_t& a, uint32_t& b) {
    const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    a = r[0];
    b = r[1];
}
__device__ __forceinline__ int pair_sum(int x) {
    uint32_t a, b;
    pair_halves((uint32_t)x, a, b);
    return (int)a + (int)b;
}
__device__ __forceinline__ float pair_min(float x) {
    uint32_t a, b;
    pair_halves(__builtin_bit_cast(uint32_t, x), a, b);
    return fminf(__builtin_bit_cast(float, a), __builtin_bit_cast(float, b));
}
__device__ __forceinline__ double pair_sum(double x) {
    const uint64_t u = __builtin_bit_cast(uint64_t, x);
    uint32_t a0, b0, a1, b1;
    pair_halves((uint32_t)u, a0, b0);
    pair_halves((uint32_t)(u >> 32), a1, b1);
    return __builtin_bit_cast(double, (uint64_t)a0 | ((uint64_t)a1 << 32)) +
           __builtin_bit_cast(double, (uint64_t)b0 | ((uint64_t)b1 << 32));
}

// OR over the 64 lanes of a wave by DPP row shifts and broadcasts, returned
// to every lane.
__device__ __forceinline__ uint32_t wave_or(uint32_t x) {
#define ENTMAX_OR_STEP(ctrl, rmask) x |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, ctrl, rmask, 0xf, false)
    ENTMAX_OR_STEP(0x111, 0xf);
    ENTMAX_OR_STEP(0x112, 0xf);
    ENTMAX_OR_STEP(0x114, 0xf);
    ENTMAX_OR_STEP(0x118, 0xf);
    ENTMAX_OR_STEP(0x142, 0xa);
    ENTMAX_OR_STEP(0x143, 0xc);
#undef ENTMAX_OR_STEP
    return (uint32_t)__builtin_amdgcn_readlane((int)x, 63);
}

// One Halley step for f(t) = F(t) - 1 with F(t) = sum [(s - t)/2]_+^2:
// f' = -F1 (F1 = sum [(s - t)/2]_+), f'' = C/2 (C = #{s > t}).
// Returns the step target, or the bracket midpoint when the step leaves
// (lo, hi) or is undefined.
__device__ __forceinline__ float halley_or_bisect(float t, float F, float F1, float C,
                                                  float lo, float hi) {
    const float f = F - 1.0f;
    const float fp = -F1;
    const float fpp = 0.5f * C;
    const float den = 2.0f * fp * fp - f * fpp;
    float tn = t - 2.0f * f * fp / den;
    if (!(den > 0.0f) || !(tn > lo && tn < hi)) tn = 0.5f * (lo + hi);
    return tn;
}

// Threshold of a fixed support from its count and the sums of y = s - m and
// y^2 (m = row max): the smaller root of C t^2 - 2 S1 t + (S2 - 4) = 0,
// returned in score units (m + t).
__device__ __forceinline__ float support_root(float m, float C, float S1, float S2) {
    const float disc = fmaxf(S1 * S1 - C * (S2 - 4.0f), 0.0f);
    return m + (S1 - sqrtf(disc)) / C;
}

// The alpha-entmax map for alpha in (1, 2] in score units ("AdaSplash-2:
// Faster Differentiable Sparse Attention" sec. 2.3, whose tau' is
// (alpha - 1) tau here):  p = [u]_+^e with u = (alpha - 1)(s - tau) and
// e = 1/(alpha - 1).  dp/ds = u^(e-1) = p/u on the support, and
// d/dtau sum p = -sum u^(e-1).  alpha = 2 (e = 1) is sparsemax, p = u.
struct AlphaMap {
    float am1;  // alpha - 1
    float e;    // 1 / (alpha - 1)
    int lin;    // alpha == 2
    __device__ __forceinline__ float pw(float u) const {
        if (!(u > 0.0f)) return 0.0f;
        return lin ? u : exp2f(e * log2f(u));
    }
    // (s > tau is tested before the difference is formed: a masked score
    // against the threshold of a row with no active key, -inf - -inf, would
    // give a NaN, and the build assumes no NaN reaches a comparison)
    __device__ __forceinline__ float p(float s, float tau) const { return s > tau ? pw(am1 * (s - tau)) : 0.0f; }
    // u^(e-1) for u > 0 (1 for sparsemax), 0 otherwise: p = u * pw1(u) and
    // p/u = pw1(u), so a Newton step needs one power and no division
    __device__ __forceinline__ float pw1(float u) const {
        if (!(u > 0.0f)) return 0.0f;
        return lin ? 1.0f : exp2f((e - 1.0f) * log2f(u));
    }
    // dp/ds = u^(e-1) on the support (1 for sparsemax), 0 off it
    __device__ __forceinline__ float g(float s, float tau) const {
        if (!(s > tau)) return 0.0f;
        const float u = am1 * (s - tau);
        if (!(u > 0.0f)) return 0.0f;
        return lin ? 1.0f : exp2f((e - 1.0f) * log2f(u));
    }
    // upper bracket end of a row of n entries with maximum m: p_max >= 1/n
    __device__ __forceinline__ float hi(float m, float n) const {
        return m - exp2f(-am1 * log2f(n)) * e;
    }
};

inline AlphaMap make_alpha_map(float alpha) {
    AlphaMap a;
    a.am1 = alpha - 1.0f;
    a.e = 1.0f / a.am1;
    a.lin = alpha == 2.0f ? 1 : 0;
    return a;
}

// Newton step from below for the alpha-entmax normaliser F = sum p = 1, with
// F1 = sum p/u = -dF/dtau, taken on g = F^(alpha-1) - 1 (the e-norm of the
// u_i, e = 1/(alpha-1), less 1) rather than on F - 1: g is convex and
// decreasing in tau like F, so from a point with g >= 0 the step stays at or
// below the root, and it is close to linear (exactly so while a single score
// is above tau), where F - 1 grows like a power e of the distance and
// Newton on it closes only 1 - 1/e of the gap per step far from the root.
// The step is e (F - F^(2-alpha)) / F1 (the plain Newton step at alpha = 2).
// From a point above the root (reached through the rounding of the sums) the
// same tangent lands at or below the root, again by convexity, so the step
// is taken from there too: a bisection from above would need a halving per
// bit of the gap left to the last point below.
// Steps that leave (lo, hi) fall back to bisection.  Returns the next point
// and updates the bracket; *done is set once the step is below 1e-6 relative
// (tau is then the returned point, one Newton step further, so its error is
// of the order of the squared step).  A tighter stop would sit at the
// rounding noise of the fp32 sums, where Newton no longer settles and only
// the iteration cap ends the loop.
__device__ __forceinline__ float newton_or_bisect(float t, float F, float F1, float& lo, float& hi,
                                                  bool* done, const AlphaMap& am) {
    *done = false;
    const float tol = 1e-6f * fmaxf(1.0f, fabsf(t));
    if (F - 1.0f >= 0.0f) {
        lo = t;
        const float Fq = am.lin ? 1.0f : exp2f((1.0f - am.am1) * log2f(F));  // F^(2-alpha)
        const float step = am.e * (F - Fq) / F1;
        const float tn = t + step;
        if (!(step > tol)) {
            *done = true;
            return fminf(fmaxf(tn, lo), hi);
        }
        return (tn < hi) ? tn : 0.5f * (lo + hi);
    }
    hi = t;
    if (F > 0.0f && F1 > 0.0f) {
        const float Fq = am.lin ? 1.0f : exp2f((1.0f - am.am1) * log2f(F));
        const float step = am.e * (F - Fq) / F1;  // < 0
        const float tn = t + step;
        if (tn > lo) {
            if (!(-step > tol)) *done = true;
            return tn;
        }
    }
    return 0.5f * (lo + hi);
}

}  // namespace entmax
