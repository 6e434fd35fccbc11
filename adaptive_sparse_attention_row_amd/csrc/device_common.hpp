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

}  // namespace entmax
