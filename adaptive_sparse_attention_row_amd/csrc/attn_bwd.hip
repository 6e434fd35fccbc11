// attn_bwd.hip -- alpha-entmax attention backward on gfx950 (written for
// alpha = 1.5 below; other alpha in (1, 2] use g = u^(1/(alpha-1) - 1),
// u = (alpha - 1)(S - tau), the derivative of A in S, in the same formulas).
//
// With g = [(S - tau)/2]_+ (so A = g^2), the threshold's implicit derivative
// gives, on the support only ("AdaSplash-2: Faster Differentiable Sparse
// Attention", sec. 3.3 "Backward pass", appendix C.6):
//   dA_ij = dO_i . V_j,   delta_i = sum_j g_ij dA_ij / sum_j g_ij,
//   dS_ij = g_ij (dA_ij - delta_i),
//   dQ = scale dS K,  dK = scale dS^T Q,  dV = A^T dO.
// Both kernels walk the forward's block mask, so null 64x64 tiles cost
// nothing (AdaSplash-2 uses M for dQ and its transpose for dK, dV).
//
// bwd_dq32  (bf16) one workgroup per 128 query rows, each wave 32 of them
//           and every listed tile of the block (lanes are queries).  Pass 1
//           over the rows' non-null tiles: S^T = K Q^T and dA^T = V dO^T on
//           MFMA, accumulating sum g dA and sum g per row -> delta (also
//           written for the dK sweep).  Pass 2: dS, then dQ^T += K^T dS^T.
// bwd_dq    (fp32) the same two passes with 64 rows per wave and the key
//           tiles split between wave pairs.
// bwd_dkdv  one workgroup per 128 keys (fp32 at d = 64: 256), lanes are
//           keys.  For every query tile of the mask column: S = Q K^T and
//           dA = dO V^T on MFMA, then dV^T += dO^T A and dK^T += Q^T dS;
//           for bf16 as two sweeps, dV (PART 1) then dK (PART 2), each
//           holding one accumulator and operand set.
// bwd_range (bf16) the largest magnitudes of Q, K, V and dO, from which
//           every workgroup derives the power-of-two scales of its fp16
//           weight products.
// Every kernel has one instance per alpha class (GEN: alpha != 1.5).
// For bf16 the products with the weights (A, dS) run on fp16 MFMA with both
// operands scaled by powers of two; for fp32 on the fp32 path of the shared
// tile operations.  Accumulation is fp32; all gradients are written in fp32.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "attn_common.hpp"
#include "device_common.hpp"
#include "launch.hpp"
#include "tile_dma.hpp"

namespace entmax {
namespace attn {
namespace {

struct BwdParams {
    const void* q;
    const void* k;
    const void* v;
    const void* dout;
    const float* tau;
    const uint32_t* mask;  // [BH][Tr64][Wd]
    float* dq;
    float* dk;
    float* dv;
    float* delta;  // workspace [BH][L]
    const float* gv;    // [BH][L][d] sum_j g V_j from the forward (null: delta from a pass over the keys)
    const float* gsum;  // [BH][L] sum_j g
    const uint32_t* range;  // workspace [kRangeBlocks][4]: max |Q|, |K|, |V|, |dO| bits per block (bf16)
    int BH, L, mode, W, nQ, nKB, Tc, Tr64, Wd;
    float scale;
    AlphaMap am;  // the alpha-entmax map
    int gen;      // alpha != 1.5
};

// The kernels are instantiated per alpha class (GEN: alpha != 1.5), and
// by_alpha<GEN>(f) hands f that class as a type.  A runtime test inside the
// per-element loops compiled to a branch per element; both paths in one
// instance cost registers (spills at d = 128).
template <bool GEN, class F>
__device__ __forceinline__ void by_alpha(F f) {
    f(std::integral_constant<bool, GEN>{});
}

// Stage one 64-row tile of X (rows r0 .., zero past L) into LDS, in the
// score-operand layout or the PV-operand layout.
template <typename T, int D>
__device__ __forceinline__ void stage_score(T* dst, const T* Xh, int r0, int L) {
    using O = Ops<T, D>;
    constexpr int kIt = (O::kChunks + kNT - 1) / kNT;
    u32x4 v[kIt];
    // (a tile wholly below L loads without the per-row bounds)
    if (r0 + kBC <= L) {
#pragma unroll
        for (int i = 0; i < kIt; ++i) {
            const int c = threadIdx.x + i * kNT;
            if (c < O::kChunks) v[i] = O::template load_k_chunk<true>(Xh, r0, L, c);
        }
    } else {
#pragma unroll
        for (int i = 0; i < kIt; ++i) {
            const int c = threadIdx.x + i * kNT;
            if (c < O::kChunks) v[i] = O::load_k_chunk(Xh, r0, L, c);
        }
    }
#pragma unroll
    for (int i = 0; i < kIt; ++i) {
        const int c = threadIdx.x + i * kNT;
        if (c < O::kChunks) O::store_k_chunk(dst, c, v[i]);
    }
}

// The same staging split in two, so that a tile's loads can be in flight
// while the previous tile is in use: its chunks in registers, then in LDS.
template <typename T, int D>
struct ScoreTileRegs {
    static constexpr int kIt = (Ops<T, D>::kChunks + kNT - 1) / kNT;
    u32x4 v[kIt];
    __device__ __forceinline__ void load(const T* Xh, int r0, int L) {
        if (r0 + kBC <= L) {
#pragma unroll
            for (int i = 0; i < kIt; ++i) {
                const int c = threadIdx.x + i * kNT;
                if (c < Ops<T, D>::kChunks) v[i] = Ops<T, D>::template load_k_chunk<true>(Xh, r0, L, c);
            }
        } else {
#pragma unroll
            for (int i = 0; i < kIt; ++i) {
                const int c = threadIdx.x + i * kNT;
                if (c < Ops<T, D>::kChunks) v[i] = Ops<T, D>::load_k_chunk(Xh, r0, L, c);
            }
        }
    }
    __device__ __forceinline__ void store(T* dst) const {
#pragma unroll
        for (int i = 0; i < kIt; ++i) {
            const int c = threadIdx.x + i * kNT;
            if (c < Ops<T, D>::kChunks) Ops<T, D>::store_k_chunk(dst, c, v[i]);
        }
    }
};

template <typename T, int D>
__device__ __forceinline__ void stage_pv(T* dst, const T* Xh, int r0, int L) {
    using O = Ops<T, D>;
    constexpr int kIt = (O::kVUnits + kNT - 1) / kNT;
    typename O::VRegs v[kIt];
    if (r0 + kBC <= L) {
#pragma unroll
        for (int i = 0; i < kIt; ++i) {
            const int u = threadIdx.x + i * kNT;
            if (u < O::kVUnits) v[i] = O::template load_v_unit<true>(Xh, r0, L, u);
        }
    } else {
#pragma unroll
        for (int i = 0; i < kIt; ++i) {
            const int u = threadIdx.x + i * kNT;
            if (u < O::kVUnits) v[i] = O::load_v_unit(Xh, r0, L, u);
        }
    }
#pragma unroll
    for (int i = 0; i < kIt; ++i) {
        const int u = threadIdx.x + i * kNT;
        if (u < O::kVUnits) O::store_v_unit(dst, u, v[i]);
    }
}

template <typename T, int D>
struct PvTileRegs {
    static constexpr int kIt = (Ops<T, D>::kVUnits + kNT - 1) / kNT;
    typename Ops<T, D>::VRegs v[kIt];
    __device__ __forceinline__ void load(const T* Xh, int r0, int L) {
        if (r0 + kBC <= L) {
#pragma unroll
            for (int i = 0; i < kIt; ++i) {
                const int u = threadIdx.x + i * kNT;
                if (u < Ops<T, D>::kVUnits) v[i] = Ops<T, D>::template load_v_unit<true>(Xh, r0, L, u);
            }
        } else {
#pragma unroll
            for (int i = 0; i < kIt; ++i) {
                const int u = threadIdx.x + i * kNT;
                if (u < Ops<T, D>::kVUnits) v[i] = Ops<T, D>::load_v_unit(Xh, r0, L, u);
            }
        }
    }
    __device__ __forceinline__ void store(T* dst) const {
#pragma unroll
        for (int i = 0; i < kIt; ++i) {
            const int u = threadIdx.x + i * kNT;
            if (u < Ops<T, D>::kVUnits) Ops<T, D>::store_v_unit(dst, u, v[i]);
        }
    }
    // The tile in fp16 times sc (bf16 only).
    __device__ __forceinline__ void store16(uint16_t* dst, float sc) const {
#pragma unroll
        for (int i = 0; i < kIt; ++i) {
            const int u = threadIdx.x + i * kNT;
            if (u < Ops<T, D>::kVUnits) Ops<T, D>::store_v_unit_f16(dst, u, v[i], sc);
        }
    }
};

// The PV-layout tile of X for the weight products: fp16 times sc for bf16
// inputs (sc a power of two), the input type itself for fp32.
template <typename T, int D>
__device__ __forceinline__ void stage_pvw(T* dst, const T* Xh, int r0, int L, float sc) {
    if constexpr (sizeof(T) == 2) {
        PvTileRegs<T, D> r;
        r.load(Xh, r0, L);
        r.store16(reinterpret_cast<uint16_t*>(dst), sc);
    } else {
        stage_pv<T, D>(dst, Xh, r0, L);
    }
}

// Direct global -> LDS staging of one 64-row tile in the score layout (the
// swizzled natural layout of store_k_chunk): each wave issues a quarter of
// the tile's 16-byte chunks; rows past L read row L - 1, whose scores the
// callers mask.  r0 (< L) must be wave-uniform.  Addresses are recomputed per
// call rather than kept in registers.
template <typename T, int D>
__device__ __forceinline__ void dma_tile(T* dst, const T* Xh, int r0, int L) {
    using DMA = TileDMA<T, D>;
    constexpr int kCPR = DMA::kCPR, kPerWave = DMA::kTileCh / 4, kIpw = kPerWave / kWave;
    constexpr int kSlot = 16 / (int)sizeof(T);
    static_assert(kPerWave % kWave == 0, "chunks per wave");
    const int w = wave_id(), lane = lane_id();
    const T* tb = Xh + (size_t)r0 * D;
#pragma unroll
    for (int k = 0; k < kIpw; ++k) {
        const int q = w * kPerWave + k * kWave + lane;
        int row = q / kCPR;
        const int col = swz<kCPR>(row, q % kCPR) * kSlot;
        row = r0 + row < L ? row : L - 1 - r0;
        __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(tb + row * D + col),
                                         (__attribute__((address_space(3))) void*)(dst + (w * kPerWave + k * kWave) * kSlot),
                                         16, 0, 0);
    }
}

// ------------------------------------------------------------ fp16 products
// For bf16 inputs the products with the weights (4A into dV, 2 dS into dK and
// dQ) run as one fp16 MFMA per block, not a bf16 hi + lo pair.  Both operands
// are scaled by powers of two, so that no product leaves fp16's range and the
// results are scaled back exactly: Q, K and dO by 2^(15 - E) where 2^E bounds
// the tensor's largest magnitude (bf16 -> fp16 is then exact down to 29
// binades below that maximum), 4A <= 4 by 2^12, and 2 dS by the same rule
// applied to its bound |2 dS| = |dd (dA - delta)| <= 4 |dA|max
// <= 4 d max|dO| max|V| (dd <= 2 on the support, delta an average of dA).
// A range pass over the inputs records the maxima; every workgroup reads
// them and derives the same scales.
constexpr int kRangeBlocks = 256;

__global__ __launch_bounds__(kNT) void bwd_range_kernel(const __bf16* q, const __bf16* k, const __bf16* v,
                                                        const __bf16* dout, size_t n, uint32_t* out) {
    __shared__ uint32_t red[4];
    if (threadIdx.x < 4) red[threadIdx.x] = 0u;
    __syncthreads();
    const __bf16* src[4] = {q, k, v, dout};
    const size_t n8 = n / 8;
#pragma unroll
    for (int a = 0; a < 4; ++a) {
        uint32_t mx = 0u;  // largest |x| as bf16 bits (monotone for finite values)
        const u32x4* p = reinterpret_cast<const u32x4*>(src[a]);
        for (size_t i = (size_t)blockIdx.x * kNT + threadIdx.x; i < n8; i += (size_t)kRangeBlocks * kNT) {
            const u32x4 x = p[i];
#pragma unroll
            for (int j = 0; j < 4; ++j) mx = max(mx, max(x[j] & 0x7fffu, (x[j] >> 16) & 0x7fffu));
        }
        if (blockIdx.x == 0 && threadIdx.x < n - n8 * 8) {
            const uint32_t b = __builtin_bit_cast(uint16_t, src[a][n8 * 8 + threadIdx.x]);
            mx = max(mx, b & 0x7fffu);
        }
        atomicMax(&red[a], mx);
    }
    __syncthreads();
    if (threadIdx.x < 4) out[blockIdx.x * 4 + threadIdx.x] = red[threadIdx.x];
}

struct F16Scales {
    float q, k, o, a, s;  // operand scales: Q, K, dO tiles; 4A and 2 dS weights
};

// The exponent E with |x| < 2^E for the bf16 bit pattern b (E = 0 for 0).
__device__ __forceinline__ int bound_exp(uint32_t b) {
    return b ? (int)((b >> 7) & 0xffu) - 126 : 0;
}

__device__ __forceinline__ float pow2(int e) {
    e = e < -60 ? -60 : (e > 60 ? 60 : e);
    return __builtin_bit_cast(float, (uint32_t)(e + 127) << 23);
}

// The scales of the fp16 products (all 1 for fp32 inputs); `red` is 4 words
// of LDS.  The same in every workgroup.  Ends with a barrier.
template <typename T, int D>
__device__ __forceinline__ F16Scales f16_scales(const BwdParams& p, uint32_t* red) {
    F16Scales f = {1.f, 1.f, 1.f, 1.f, 1.f};
    if constexpr (sizeof(T) == 2) {
        if (threadIdx.x < 4) red[threadIdx.x] = 0u;
        __syncthreads();
        if (threadIdx.x < kRangeBlocks) {
#pragma unroll
            for (int a = 0; a < 4; ++a) atomicMax(&red[a], p.range[threadIdx.x * 4 + a]);
        }
        __syncthreads();
        constexpr int kLogD = D == 128 ? 7 : 6;
        const int eq = bound_exp(red[0]), ek = bound_exp(red[1]), ev = bound_exp(red[2]), eo = bound_exp(red[3]);
        f.q = pow2(15 - eq);
        f.k = pow2(15 - ek);
        f.o = pow2(15 - eo);
        f.a = 4096.0f;
        f.s = pow2(15 - (eo + ev + 2 + kLogD));
        __syncthreads();
    }
    return f;
}

// The weight product for the tile type: fp16 with weight scale ws for bf16
// (the tile staged by stage_pvw), the fp32 product for fp32.
template <typename T, int D, int NB>
__device__ __forceinline__ void pv_w(typename Ops<T, D>::template OAcc<NB>& oa, const T* Vt,
                                     const f32x16 (&a)[2][NB], const bool (&on)[2], float ws) {
    if constexpr (sizeof(T) == 2)
        Ops<T, D>::template pv_f16<NB>(oa, reinterpret_cast<const uint16_t*>(Vt), a, on, ws);
    else
        Ops<T, D>::template pv<NB>(oa, Vt, a, on);
}

template <class FlagsOf>
__device__ __forceinline__ int build_list16(uint16_t* list, int n_items, FlagsOf flags_of) {
    const int l = lane_id();
    int n = 0;
    for (int base = 0; base < n_items; base += kWave) {
        const int J = base + l;
        const int f = (J < n_items) ? flags_of(J) : 0;
        const uint64_t b = __ballot(f != 0);
        if (f) list[n + lanes_below(b)] = (uint16_t)(J | (f << 12));
        n += __popcll(b);
    }
    return n;
}

// Tiles staged per step by the dQ kernel: 2 (one per key-parity wave pair),
// or 1 when LDS cannot hold two (fp32, d = 128).
template <typename T, int D>
struct DqCfg {
    static constexpr int kTps = (sizeof(T) == 4 && D == 128) ? 1 : 2;
    static constexpr int kBlk = Ops<T, D>::kKTile > Ops<T, D>::kVTile ? Ops<T, D>::kKTile : Ops<T, D>::kVTile;
};

// ------------------------------------------------------------ delta from G.V
// delta_i = sum_j g_ij dA_ij / sum_j g_ij = dO_i . (sum_j g_ij V_j) / sum_j g_ij:
// with G.V and sum g from the forward, one dot product per row.  D / 8 lanes
// per row (an aligned group of a wave), each with 8 elements of d (one
// 16-byte load of dO); the grid strides over the rows.
template <typename T, int D>
__global__ __launch_bounds__(kNT) void bwd_delta_kernel(BwdParams p) {
    constexpr int kLpr = D / 8;  // lanes per row
    const size_t rows = (size_t)p.BH * p.L;
    const size_t stride = (size_t)gridDim.x * (kNT / kLpr);
    const int part = threadIdx.x % kLpr;
    for (size_t row = (size_t)blockIdx.x * (kNT / kLpr) + threadIdx.x / kLpr; row < rows; row += stride) {
        float acc = 0.0f;
        const T* dO = reinterpret_cast<const T*>(p.dout) + row * D + part * 8;
        const float* gv = p.gv + row * D + part * 8;
        const f32x4 g0 = *reinterpret_cast<const f32x4*>(gv), g1 = *reinterpret_cast<const f32x4*>(gv + 4);
        if constexpr (sizeof(T) == 2) {
            const u32x4 x = *reinterpret_cast<const u32x4*>(dO);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float o = __builtin_bit_cast(float, ((x[e >> 1] >> ((e & 1) * 16)) & 0xffffu) << 16);
                acc = fmaf(o, e < 4 ? g0[e] : g1[e - 4], acc);
            }
        } else {
            const f32x4 o0 = *reinterpret_cast<const f32x4*>(dO), o1 = *reinterpret_cast<const f32x4*>(dO + 4);
#pragma unroll
            for (int e = 0; e < 4; ++e) acc = fmaf(o0[e], g0[e], fmaf(o1[e], g1[e], acc));
        }
#pragma unroll
        for (int o = kLpr / 2; o > 0; o >>= 1) acc += __shfl_xor(acc, o, kWave);
        if (part == 0) {
            const float den = p.gsum[row];
            p.delta[row] = den > 0.0f ? acc / den : 0.0f;
        }
    }
}

// ------------------------------------------------------------ dQ kernel
template <typename T, int D, bool GEN>
__global__ __launch_bounds__(kNT, 1) void bwd_dq_kernel(BwdParams p) {
    using O = Ops<T, D>;
    constexpr int TPS = DqCfg<T, D>::kTps;
    constexpr int BLK = DqCfg<T, D>::kBlk;
    constexpr int kRed = 2 * 64 * (D + 4);
    constexpr int kStage = TPS * 3 * BLK * (int)sizeof(T);
    constexpr int kBytes = kStage > kRed * 4 ? kStage : kRed * 4;
    __shared__ __attribute__((aligned(16))) unsigned char smem[kBytes];
    __shared__ uint16_t list[kMaxTc];
    __shared__ uint32_t mw[2][kMaxTc / 32];
    __shared__ float part[2][kBR][2];
    __shared__ int nlist_s;
    T* lds = reinterpret_cast<T*>(smem);

    const int t = threadIdx.x, w = wave_id(), qh = w & 1, kh = w >> 1;
    const int l = lane_id(), m = l & 31, h = l >> 5;
    int bh, r0;
    decode_item(blockIdx.x, p.BH, p.nQ, p.mode != 0, bh, r0);
    const int R0 = r0 + 64 * qh;
    const Geom g = {p.L, p.mode, p.W};
    const size_t head_off = (size_t)bh * p.L * D;
    const T* Qh = reinterpret_cast<const T*>(p.q) + head_off;
    const T* Kh = reinterpret_cast<const T*>(p.k) + head_off;
    const T* Vh = reinterpret_cast<const T*>(p.v) + head_off;
    const T* dOh = reinterpret_cast<const T*>(p.dout) + head_off;

    for (int i = t; i < 2 * p.Wd; i += kNT) {
        const int hh = i / p.Wd, wd = i % p.Wd;
        const int I = r0 / 64 + hh;
        mw[hh][wd] = (I < p.Tr64) ? p.mask[((size_t)bh * p.Tr64 + I) * p.Wd + wd] : 0u;
    }
    __syncthreads();
    if (w == 0) {
        const int n = build_list16(list, p.Tc, [&](int J) {
            return (int)((mw[0][J >> 5] >> (J & 31)) & 1u) | (int)(((mw[1][J >> 5] >> (J & 31)) & 1u) << 1);
        });
        if (l == 0) nlist_s = n;
    }
    typename O::template QOp<2> qop, dop;
    O::load_q(qop, Qh, R0, p.L);
    O::load_q(dop, dOh, R0, p.L);
    float tq[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        const int row = R0 + qb * 32 + m;
        tq[qb] = (row < p.L) ? p.tau[(size_t)bh * p.L + row] : __builtin_inff();
    }
    __syncthreads();
    const int n = nlist_s;

    // Walk the list; fn(J, Kt, Vt, KPVt) for each tile flagged for this half
    // (K in the PV layout staged only when the pass takes the product with K).
    auto walk = [&](auto with_pv, auto fn) {
        const int steps = (n + TPS - 1) / TPS;
        for (int st = 0; st < steps; ++st) {
            __syncthreads();
#pragma unroll
            for (int u = 0; u < TPS; ++u) {
                const int e = st * TPS + u;
                const int J = (e < n) ? (list[e] & 0xfff) : 0;
                const int c0 = (e < n) ? J * kBC : p.L;
                T* base = lds + u * 3 * BLK;
                stage_score<T, D>(base, Kh, c0, p.L);
                stage_score<T, D>(base + BLK, Vh, c0, p.L);
                if constexpr (decltype(with_pv)::value) stage_pv<T, D>(base + 2 * BLK, Kh, c0, p.L);
            }
            __syncthreads();
            const int u = (TPS == 2) ? kh : 0;
            const int e = st * TPS + u;
            if (e >= n || (TPS == 1 && (st & 1) != kh)) continue;
            const int ent = list[e];
            if (!((ent >> (12 + qh)) & 1)) continue;
            const int J = ent & 0xfff;
            const int cls = tile_class(J, R0, g);
            if (cls == kSkip) continue;
            const T* base = lds + u * 3 * BLK;
            fn(J, cls, base, base + BLK, base + 2 * BLK);
        }
        __syncthreads();
    };

    // ---- pass 1: delta_i = sum g dA / sum g  (2g used on both sides)
    float num[2] = {0.f, 0.f}, den[2] = {0.f, 0.f};
    walk(std::false_type{}, [&](int J, int cls, const T* Kt, const T* Vt, const T*) {
        f32x16 s[2][2], da[2][2];
        O::scores(s, Kt, qop);
        if (cls == kPartial) apply_mask(s, J, R0, g);
        O::scores(da, Vt, dop);
        by_alpha<GEN>([&](auto gen_c) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int qb = 0; qb < 2; ++qb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const float sv = s[kb][qb][r] * p.scale;
                        const float dd = gen_c ? 2.0f * p.am.g(sv, tq[qb]) : fmaxf(sv - tq[qb], 0.0f);
                        num[qb] += dd * da[kb][qb][r];
                        den[qb] += dd;
                    }
        });
    });
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        num[qb] += __shfl_xor(num[qb], 32, kWave);
        den[qb] += __shfl_xor(den[qb], 32, kWave);
        if (h == 0) {
            part[kh][qh * 64 + qb * 32 + m][0] = num[qb];
            part[kh][qh * 64 + qb * 32 + m][1] = den[qb];
        }
    }
    __syncthreads();
    float dl[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        const int rr = qh * 64 + qb * 32 + m;
        const float nn = part[0][rr][0] + part[1][rr][0];
        const float dn = part[0][rr][1] + part[1][rr][1];
        dl[qb] = dn > 0.f ? nn / dn : 0.f;
        const int row = r0 + rr;
        if (kh == 0 && h == 0 && row < p.L) p.delta[(size_t)bh * p.L + row] = dl[qb];
    }

    // ---- pass 2: dQ^T += K^T (2 dS)^T
    typename O::template OAcc<2> oa;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
#pragma unroll
            for (int i = 0; i < 16; ++i) oa.o[db][qb][i] = 0.f;
    walk(std::true_type{}, [&](int J, int cls, const T* Kt, const T* Vt, const T* KPVt) {
        f32x16 s[2][2], da[2][2];
        O::scores(s, Kt, qop);
        if (cls == kPartial) apply_mask(s, J, R0, g);
        O::scores(da, Vt, dop);
        by_alpha<GEN>([&](auto gen_c) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int qb = 0; qb < 2; ++qb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const float sv = s[kb][qb][r] * p.scale;
                        const float dd = gen_c ? 2.0f * p.am.g(sv, tq[qb]) : fmaxf(sv - tq[qb], 0.0f);
                        s[kb][qb][r] = dd * (da[kb][qb][r] - dl[qb]);
                    }
        });
        const bool on[2] = {true, true};
        O::pv(oa, KPVt, s, on);
    });

    float* red = reinterpret_cast<float*>(smem);
    constexpr int kRS = D + 4;
    if (kh == 1) {
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int qb = 0; qb < 2; ++qb)
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4) {
                    f32x4 v4;
#pragma unroll
                    for (int e = 0; e < 4; ++e) v4[e] = oa.o[db][qb][4 * r4 + e];
                    *reinterpret_cast<f32x4*>(red + (qh * 64 + qb * 32 + m) * kRS + db * 32 + 8 * r4 + 4 * h) = v4;
                }
    }
    __syncthreads();
    if (kh == 0) {
        const float f = 0.5f * p.scale;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
                const int q = qb * 32 + m;
                const int row = R0 + q;
                if (row >= p.L) continue;
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4) {
                    const int d = db * 32 + 8 * r4 + 4 * h;
                    const f32x4 o2 = *reinterpret_cast<const f32x4*>(red + (qh * 64 + q) * kRS + d);
                    f32x4 v4;
#pragma unroll
                    for (int e = 0; e < 4; ++e) v4[e] = f * (oa.o[db][qb][4 * r4 + e] + o2[e]);
                    *reinterpret_cast<f32x4*>(p.dq + ((size_t)bh * p.L + row) * D + d) = v4;
                }
            }
    }
}

// ------------------------------------------------------------ dQ kernel, bf16
// The same two passes with 32 query rows per wave: the four waves of a
// workgroup take the 128 rows in quarters and every one of them walks all of
// the block's listed tiles, so each wave sums over all keys of its rows (no
// reduction across waves) and holds half the operands and accumulators of
// the layout above.  That fits two workgroups per CU (one wave's staging
// then overlaps another's products) where the layout above runs one.
template <int D, bool GEN>
__global__ __launch_bounds__(kNT, 2) void bwd_dq32_kernel(BwdParams p) {
    using T = __bf16;
    using O = Ops<T, D>;
    constexpr int BLK = DqCfg<T, D>::kBlk;
    __shared__ __attribute__((aligned(16))) T lds[3 * BLK];
    __shared__ uint16_t list[kMaxTc];
    __shared__ uint32_t mw[2][kMaxTc / 32];
    __shared__ uint32_t red[4];
    __shared__ int nlist_s;

    const int t = threadIdx.x, w = wave_id();
    const int l = lane_id(), m = l & 31, h = l >> 5;
    int bh, r0;
    decode_item(blockIdx.x, p.BH, p.nQ, p.mode != 0, bh, r0);
    const F16Scales fs = f16_scales<T, D>(p, red);
    const int R0 = r0 + 32 * w;  // this wave's rows
    const int half = w >> 1;     // their 64-row block
    const Geom g = {p.L, p.mode, p.W};
    const size_t head_off = (size_t)bh * p.L * D;
    const T* Qh = reinterpret_cast<const T*>(p.q) + head_off;
    const T* Kh = reinterpret_cast<const T*>(p.k) + head_off;
    const T* Vh = reinterpret_cast<const T*>(p.v) + head_off;
    const T* dOh = reinterpret_cast<const T*>(p.dout) + head_off;

    for (int i = t; i < 2 * p.Wd; i += kNT) {
        const int hh = i / p.Wd, wd = i % p.Wd;
        const int I = r0 / 64 + hh;
        mw[hh][wd] = (I < p.Tr64) ? p.mask[((size_t)bh * p.Tr64 + I) * p.Wd + wd] : 0u;
    }
    __syncthreads();
    if (w == 0) {
        const int n = build_list16(list, p.Tc, [&](int J) {
            return (int)((mw[0][J >> 5] >> (J & 31)) & 1u) | (int)(((mw[1][J >> 5] >> (J & 31)) & 1u) << 1);
        });
        if (l == 0) nlist_s = n;
    }
    typename O::template QOp<1> qop, dop;
    O::load_q(qop, Qh, R0, p.L);
    O::load_q(dop, dOh, R0, p.L);
    const int row = R0 + m;
    const float tq = (row < p.L) ? p.tau[(size_t)bh * p.L + row] : __builtin_inff();
    __syncthreads();
    const int n = nlist_s;

    // Walk the listed tiles.  K and V in the score layout go to LDS by
    // direct global -> LDS loads, issued for the next tile as soon as every
    // wave has taken its score products from the current one; the K tile in
    // the PV layout (fp16, scaled), which the dQ pass needs, is loaded into
    // registers while the score products run and converted into LDS after
    // them (registers for a whole step ahead are not free at d = 128).  fa(J, cls, s, da) takes the products from the score tiles,
    // fc(J, cls, s, da) the rest; both run only for tiles that are non-null
    // for this wave's 64-row block and not masked out for its rows (every
    // wave takes part in the barriers).  DMA rows past L repeat row L - 1:
    // their scores are masked, so their weights are zero.
    T* const kbuf = lds;
    T* const vbuf = lds + BLK;
    T* const kpv = lds + 2 * BLK;
    auto walk = [&](auto with_pv, auto fa, auto fc) {
        constexpr bool kPv = decltype(with_pv)::value;
        PvTileRegs<T, D> rkp;
        auto issue = [&](int e) {
            const int r0 = (__builtin_amdgcn_readfirstlane(list[e]) & 0xfff) * kBC;
            dma_tile<T, D>(kbuf, Kh, r0, p.L);
            dma_tile<T, D>(vbuf, Vh, r0, p.L);
        };
        if (n > 0) issue(0);
        for (int e = 0; e < n; ++e) {
            const int ent = list[e];
            const int J = ent & 0xfff;
            wait_vmcnt<0>();
            __syncthreads();
            if constexpr (kPv) rkp.load(Kh, J * kBC, p.L);
            const int cls = ((ent >> (12 + half)) & 1) ? block_class(R0, 32, J * kBC, kBC, g) : kSkip;
            f32x16 sc[2][1], da[2][1];
            if (cls != kSkip) fa(J, cls, sc, da);
            if constexpr (kPv) rkp.store16(reinterpret_cast<uint16_t*>(kpv), fs.k);
            __syncthreads();
            if (e + 1 < n) issue(e + 1);
            if (cls != kSkip) fc(J, cls, sc, da);
        }
        __syncthreads();
    };
    // 2g (so that the factor cancels in delta), the derivative of A in S
    auto dd_of = [&](auto gen_c, float sv) { return gen_c ? 2.0f * p.am.g(sv, tq) : fmaxf(sv - tq, 0.0f); };

    // the products from the score-layout tiles (both passes)
    auto score_products = [&](int J, int cls, f32x16(&s)[2][1], f32x16(&da)[2][1]) {
        O::template scores<1>(s, kbuf, qop);
        if (cls == kPartial) apply_mask<1>(s, J, R0, g);
        O::template scores<1>(da, vbuf, dop);
    };

    // ---- pass 1: delta_i = sum g dA / sum g (given by bwd_delta_kernel when
    // the forward wrote G.V and sum g)
    float dl;
    if (p.gv != nullptr) {
        dl = row < p.L ? p.delta[(size_t)bh * p.L + row] : 0.f;
    } else {
        float num = 0.f, den = 0.f;
        walk(std::false_type{}, score_products, [&](int, int, f32x16(&s)[2][1], f32x16(&da)[2][1]) {
            by_alpha<GEN>([&](auto gen_c) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const float dd = dd_of(gen_c, s[kb][0][r] * p.scale);
                        num += dd * da[kb][0][r];
                        den += dd;
                    }
            });
        });
        num += __shfl_xor(num, 32, kWave);
        den += __shfl_xor(den, 32, kWave);
        dl = den > 0.f ? num / den : 0.f;
        if (h == 0 && row < p.L) p.delta[(size_t)bh * p.L + row] = dl;
    }

    // ---- pass 2: dQ^T += K^T (2 dS)^T
    typename O::template OAcc<1> oa;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) oa.o[db][0][i] = 0.f;
    walk(std::true_type{}, score_products, [&](int, int, f32x16(&s)[2][1], f32x16(&da)[2][1]) {
        by_alpha<GEN>([&](auto gen_c) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) s[kb][0][r] = dd_of(gen_c, s[kb][0][r] * p.scale) * (da[kb][0][r] - dl);
        });
        const bool on[2] = {true, true};
        pv_w<T, D, 1>(oa, kpv, s, on, fs.s);
    });

    if (row < p.L) {
        const float f = 0.5f * p.scale / fs.s / fs.k;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                f32x4 v4;
#pragma unroll
                for (int e = 0; e < 4; ++e) v4[e] = f * oa.o[db][0][4 * r4 + e];
                *reinterpret_cast<f32x4*>(p.dq + ((size_t)bh * p.L + row) * D + db * 32 + 8 * r4 + 4 * h) = v4;
            }
    }
}

// ------------------------------------------------------------ dK/dV kernel
template <typename T, int D>
struct DkvCfg {
    // 32-key blocks per wave (one in the split bf16 kernels, which keep two
    // workgroups per CU)
    static constexpr int kNBK = (D == 64 && sizeof(T) == 4) ? 2 : 1;
    static constexpr int kKW = 32 * kNBK;            // keys per wave
    static constexpr int kKeys = 4 * kKW;            // keys per workgroup
    static constexpr int kBlk = DqCfg<T, D>::kBlk;
};

// PART: 0 both gradients in one sweep; 1 dV only; 2 dK only.  The split
// pair recomputes S once more but each half holds one accumulator and one
// set of operands, which fits two workgroups per CU (bf16) where the joint
// kernel runs one.
template <typename T, int D, int PART, bool GEN>
__global__ __launch_bounds__(kNT, PART == 0 ? 1 : 2) void bwd_dkdv_kernel(BwdParams p) {
    using O = Ops<T, D>;
    constexpr bool kDV = PART != 2, kDK = PART != 1;
    constexpr int NBK = DkvCfg<T, D>::kNBK;
    constexpr int KW = DkvCfg<T, D>::kKW;
    constexpr int BLK = DkvCfg<T, D>::kBlk;
    __shared__ __attribute__((aligned(16))) T lds[4 * BLK];
    __shared__ uint16_t list[kMaxTc];
    __shared__ float tau_s[64], del_s[64];
    __shared__ uint32_t red[4];
    __shared__ int nlist_s;

    const int t = threadIdx.x, w = wave_id();
    const int l = lane_id(), m = l & 31, h = l >> 5;
    const F16Scales fs = f16_scales<T, D>(p, red);
    const int bh = blockIdx.x % p.BH;
    const int c0 = (blockIdx.x / p.BH) * DkvCfg<T, D>::kKeys;
    const int cw = c0 + w * KW;  // this wave's first key
    const Geom g = {p.L, p.mode, p.W};
    const size_t head_off = (size_t)bh * p.L * D;
    const T* Qh = reinterpret_cast<const T*>(p.q) + head_off;
    const T* Kh = reinterpret_cast<const T*>(p.k) + head_off;
    const T* Vh = reinterpret_cast<const T*>(p.v) + head_off;
    const T* dOh = reinterpret_cast<const T*>(p.dout) + head_off;
    const uint32_t* Mh = p.mask + (size_t)bh * p.Tr64 * p.Wd;

    // query tiles of the mask columns of the four waves' key tiles
    if (w == 0) {
        const int n = build_list16(list, p.Tr64, [&](int I) {
            int f = 0;
#pragma unroll
            for (int ww = 0; ww < 4; ++ww) {
                const int cww = c0 + ww * KW;
                if (cww < p.L) {
                    const int J = cww / kBC;
                    f |= (int)((Mh[(size_t)I * p.Wd + (J >> 5)] >> (J & 31)) & 1u) << ww;
                }
            }
            return f;
        });
        if (l == 0) nlist_s = n;
    }
    typename O::template QOp<NBK> kop, vop;
    O::load_q(kop, Kh, cw, p.L);
    if constexpr (kDK) O::load_q(vop, Vh, cw, p.L);
    typename O::template OAcc<NBK> dka, dva;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int cb = 0; cb < NBK; ++cb)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                if constexpr (kDK) dka.o[db][cb][i] = 0.f;
                if constexpr (kDV) dva.o[db][cb][i] = 0.f;
            }
    __syncthreads();
    const int n = nlist_s;
    T* Qt = lds;
    T* dOt = lds + BLK;
    T* QPVt = lds + 2 * BLK;
    T* dOPVt = lds + 3 * BLK;

    // The bf16 sweeps (PART 1, 2) stage the score-layout tiles (Q, and dO for
    // dK) by direct global -> LDS loads, issued for the next query tile as
    // soon as every wave has taken its score products from the current one;
    // the sweep's PV-layout tile (dO for dV, Q for dK; fp16, scaled) goes
    // through registers: in the dV sweep it is loaded a whole step ahead
    // (there are registers for it), in the dK sweep while the score products
    // run, and converted into LDS after them.  DMA rows past L repeat row L - 1: their tau is
    // +inf, so their weights are zero.  The fp32 joint sweep (PART 0) stages
    // synchronously.
    constexpr bool kDma = PART != 0;
    PvTileRegs<T, D> rpv;
    T* const pvt = PART == 1 ? dOPVt : QPVt;
    auto issue = [&](int e) {
        const int r0 = (__builtin_amdgcn_readfirstlane(list[e]) & 0xfff) * 64;
        dma_tile<T, D>(Qt, Qh, r0, p.L);
        if constexpr (kDK) dma_tile<T, D>(dOt, dOh, r0, p.L);
        if constexpr (PART == 1) rpv.load(dOh, r0, p.L);
    };
    if (kDma && n > 0) issue(0);
    for (int e = 0; e < n; ++e) {
        const int ent = list[e];
        const int I = ent & 0xfff;
        const int i0 = I * 64;
        if constexpr (kDma) {
            wait_vmcnt<0>();
            __syncthreads();
            if constexpr (PART == 1) {
                if constexpr (sizeof(T) == 2) rpv.store16(reinterpret_cast<uint16_t*>(pvt), fs.o);
            } else {
                rpv.load(Qh, i0, p.L);
            }
        } else {
            __syncthreads();
            stage_score<T, D>(Qt, Qh, i0, p.L);
            if constexpr (kDK) {
                stage_score<T, D>(dOt, dOh, i0, p.L);
                stage_pvw<T, D>(QPVt, Qh, i0, p.L, fs.q);
            }
            if constexpr (kDV) stage_pvw<T, D>(dOPVt, dOh, i0, p.L, fs.o);
        }
        if (t < 64) {
            const int row = i0 + t;
            tau_s[t] = (row < p.L) ? p.tau[(size_t)bh * p.L + row] : __builtin_inff();
            if constexpr (kDK) del_s[t] = (row < p.L) ? p.delta[(size_t)bh * p.L + row] : 0.f;
        }
        if constexpr (!kDma) __syncthreads();
        const int cls = ((ent >> (12 + w)) & 1) ? block_class(i0, 64, cw, KW, g) : kSkip;
        f32x16 s[2][NBK], da[2][NBK];
        if (cls != kSkip) {
            O::scores(s, Qt, kop);   // rows: queries (registers), lanes: keys
            if (cls == kPartial) apply_mask_rows_are_queries(s, i0, cw, g);
            if constexpr (kDK) O::scores(da, dOt, vop);
        }
        if constexpr (kDma) {
            if constexpr (PART == 2 && sizeof(T) == 2) rpv.store16(reinterpret_cast<uint16_t*>(pvt), fs.q);
            __syncthreads();
            if (e + 1 < n) issue(e + 1);
        }
        if (cls == kSkip) continue;
        const bool on[2] = {true, true};
        if constexpr (kDV) {
            // 4A (dd^2 with dd = 2g at alpha = 1.5), into dV
            f32x16 a4[2][NBK];
            by_alpha<GEN>([&](auto gen_c) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int cb = 0; cb < NBK; ++cb)
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const float sv = s[kb][cb][r] * p.scale;
                            const float tr = tau_s[kb * 32 + key_of_reg(r, h)];
                            if constexpr (decltype(gen_c)::value) {
                                a4[kb][cb][r] = 4.0f * p.am.p(sv, tr);
                            } else {
                                const float dd = fmaxf(sv - tr, 0.0f);
                                a4[kb][cb][r] = dd * dd;
                            }
                        }
            });
            pv_w<T, D, NBK>(dva, dOPVt, a4, on, fs.a);
        }
        if constexpr (kDK) {
            // 2 dS = dd (dA - delta) in place of S, into dK
            by_alpha<GEN>([&](auto gen_c) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int cb = 0; cb < NBK; ++cb)
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const int qi = kb * 32 + key_of_reg(r, h);
                            const float sv = s[kb][cb][r] * p.scale;
                            const float tr = tau_s[qi];
                            const float dd = gen_c ? 2.0f * p.am.g(sv, tr) : fmaxf(sv - tr, 0.0f);
                            s[kb][cb][r] = dd * (da[kb][cb][r] - del_s[qi]);
                        }
            });
            pv_w<T, D, NBK>(dka, QPVt, s, on, fs.s);
        }
    }

    const float fk = 0.5f * p.scale / fs.s / fs.q, fv = 0.25f / fs.a / fs.o;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int cb = 0; cb < NBK; ++cb) {
            const int key = cw + cb * 32 + m;
            if (key >= p.L) continue;
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                const int d = db * 32 + 8 * r4 + 4 * h;
                f32x4 k4, v4;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    if constexpr (kDK) k4[e] = fk * dka.o[db][cb][4 * r4 + e];
                    if constexpr (kDV) v4[e] = fv * dva.o[db][cb][4 * r4 + e];
                }
                if constexpr (kDK) *reinterpret_cast<f32x4*>(p.dk + ((size_t)bh * p.L + key) * D + d) = k4;
                if constexpr (kDV) *reinterpret_cast<f32x4*>(p.dv + ((size_t)bh * p.L + key) * D + d) = v4;
            }
        }
}

template <typename T, int D, bool GEN>
hipError_t launch_bwd_class(const BwdParams& bp, hipStream_t stream) {
    if constexpr (sizeof(T) == 2) {
        const size_t n = (size_t)bp.BH * bp.L * D;
        hipLaunchKernelGGL(bwd_range_kernel, dim3(kRangeBlocks), dim3(kNT), 0, stream,
                           reinterpret_cast<const __bf16*>(bp.q), reinterpret_cast<const __bf16*>(bp.k),
                           reinterpret_cast<const __bf16*>(bp.v), reinterpret_cast<const __bf16*>(bp.dout), n,
                           const_cast<uint32_t*>(bp.range));
        hipError_t e0 = hipGetLastError();
        if (e0 != hipSuccess) return e0;
    }
    if (bp.gv != nullptr) {
        const size_t blocks = ((size_t)bp.BH * bp.L * (D / 8) + kNT - 1) / kNT;
        hipLaunchKernelGGL((bwd_delta_kernel<T, D>), dim3((unsigned)(blocks < (1u << 20) ? blocks : (1u << 20))),
                           dim3(kNT), 0, stream, bp);
        hipError_t e1 = hipGetLastError();
        if (e1 != hipSuccess) return e1;
    }
    if constexpr (sizeof(T) == 2)
        hipLaunchKernelGGL((bwd_dq32_kernel<D, GEN>), dim3(bp.nQ * bp.BH), dim3(kNT), 0, stream, bp);
    else
        hipLaunchKernelGGL((bwd_dq_kernel<T, D, GEN>), dim3(bp.nQ * bp.BH), dim3(kNT), 0, stream, bp);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if constexpr (sizeof(T) == 2) {
        hipLaunchKernelGGL((bwd_dkdv_kernel<T, D, 1, GEN>), dim3(bp.nKB * bp.BH), dim3(kNT), 0, stream, bp);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL((bwd_dkdv_kernel<T, D, 2, GEN>), dim3(bp.nKB * bp.BH), dim3(kNT), 0, stream, bp);
    } else {
        hipLaunchKernelGGL((bwd_dkdv_kernel<T, D, 0, GEN>), dim3(bp.nKB * bp.BH), dim3(kNT), 0, stream, bp);
    }
    return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_bwd_typed(const BwdParams& bp, hipStream_t stream) {
    return bp.gen ? launch_bwd_class<T, D, true>(bp, stream) : launch_bwd_class<T, D, false>(bp, stream);
}

}  // namespace
}  // namespace attn

size_t attn_bwd_workspace_bytes(int B, int H, int L, int, int) {
    // delta per row, then the range pass's per-block maxima
    return (((size_t)B * H * L * sizeof(float) + 255) & ~(size_t)255) + attn::kRangeBlocks * 4 * sizeof(uint32_t);
}

hipError_t launch_attn_bwd(const AttnArgs& a, hipStream_t stream) {
    using namespace attn;
    if (a.L > kMaxL) return hipErrorInvalidValue;
    BwdParams bp;
    bp.q = a.q; bp.k = a.k; bp.v = a.v; bp.dout = a.dout;
    bp.tau = a.tau; bp.mask = a.block_mask;
    bp.dq = a.dq; bp.dk = a.dk; bp.dv = a.dv;
    bp.delta = reinterpret_cast<float*>(a.workspace);
    bp.gv = a.gv;
    bp.gsum = a.gsum;
    bp.range = reinterpret_cast<const uint32_t*>(reinterpret_cast<char*>(a.workspace) +
                                                 (((size_t)a.B * a.H * a.L * sizeof(float) + 255) & ~(size_t)255));
    bp.BH = a.B * a.H; bp.L = a.L; bp.mode = a.mask;
    bp.W = a.window < a.L ? a.window : a.L;  // a window of L or more is plain causal
    bp.nQ = (a.L + kBR - 1) / kBR;
    bp.Tc = (a.L + kBC - 1) / kBC;
    bp.Tr64 = (a.L + 63) / 64;
    bp.Wd = (bp.Tc + 31) / 32;
    bp.scale = a.scale;
    bp.am = make_alpha_map(a.alpha);
    bp.gen = a.alpha != 1.5f ? 1 : 0;
    if (a.dtype == 1) {
        if (a.d == 64) {
            bp.nKB = (a.L + DkvCfg<__bf16, 64>::kKeys - 1) / DkvCfg<__bf16, 64>::kKeys;
            return launch_bwd_typed<__bf16, 64>(bp, stream);
        }
        bp.nKB = (a.L + DkvCfg<__bf16, 128>::kKeys - 1) / DkvCfg<__bf16, 128>::kKeys;
        return launch_bwd_typed<__bf16, 128>(bp, stream);
    }
    if (a.d == 64) {
        bp.nKB = (a.L + DkvCfg<float, 64>::kKeys - 1) / DkvCfg<float, 64>::kKeys;
        return launch_bwd_typed<float, 64>(bp, stream);
    }
    bp.nKB = (a.L + DkvCfg<float, 128>::kKeys - 1) / DkvCfg<float, 128>::kKeys;
    return launch_bwd_typed<float, 128>(bp, stream);
}

}  // namespace entmax
