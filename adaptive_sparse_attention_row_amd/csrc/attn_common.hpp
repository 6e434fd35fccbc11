// attn_common.hpp -- tiles, MFMA score blocks and masks shared by the
// attention kernels (gfx950, wave64).
//
// A workgroup owns 128 query rows of one (batch, head) and runs 4 waves:
// wave w has row half qh = w & 1 (64 rows) and key parity kh = w >> 1 (it
// takes every other 64-key tile of a tile list).  Scores are computed
// transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16 (or the fp32
// 32x32x2 form), so that lane l of a 32x32 block holds query column l % 32
// and 16 keys: register r of a block holds key 8*(r/4) + 4*(l/32) + r%4.
// Per-query reductions are then lane-local plus one exchange with lane l^32.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <climits>

#include "device_common.hpp"

namespace entmax {
namespace attn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

constexpr int kBR = 128;      // query rows per workgroup
constexpr int kBC = 64;       // keys per tile
constexpr int kNT = 256;      // threads per workgroup
constexpr int kMaxTc = 1024;  // key tiles per row (L <= 65536)
constexpr int kMaxL = kMaxTc * kBC;

enum TileClass { kSkip = 0, kFull = 1, kPartial = 2 };

struct Geom {
    int L, mode, W;
};

// Classify the 64x64 tile (rows [i0, i0+64), keys of tile J) under the mask.
__device__ __forceinline__ int tile_class(int J, int i0, const Geom& g) {
    const int c0 = J * kBC, c1 = c0 + kBC - 1, i1 = i0 + 63;
    if (c0 >= g.L || i0 >= g.L) return kSkip;
    if (g.mode >= 1 && c0 > i1) return kSkip;
    if (g.mode == 2 && J != 0 && i0 - c1 > g.W) return kSkip;
    bool full = (c1 < g.L) && (i1 < g.L);
    if (g.mode >= 1) full = full && (c1 <= i0);
    if (g.mode == 2) full = full && (i1 - c0 <= g.W);
    return full ? kFull : kPartial;
}

// Active-key predicate, branch-free (it is evaluated per score element).
__device__ __forceinline__ bool key_active(int i, int j, const Geom& g) {
    const bool in_range = (i < g.L) & (j < g.L);
    const bool causal_ok = (j <= i);
    const bool window_ok = (j == 0) | (i - j <= g.W);
    const bool mode_ok = (g.mode == 0) | (causal_ok & ((g.mode == 1) | window_ok));
    return in_range & mode_ok;
}

// Key index (within a 32-key block) held by register r of lane half h.
__device__ __forceinline__ int key_of_reg(int r, int h) { return 8 * (r >> 2) + 4 * h + (r & 3); }

// Natural-layout tiles in LDS are stored unpadded with the 16-byte chunks of
// each row XOR-swizzled: chunk c of row r sits at position c ^ f(r).  With 8
// chunks per row (bf16, d = 64) f(r) = (r & 7) ^ ((r >> 3) & 1); with 16 or
// more, f(r) = r & 15.  Either way the 16-byte operand reads of 16
// consecutive rows at one chunk hit distinct bank groups (32 or 64 banks),
// and the layout can be filled by direct global->LDS loads, which write 64
// consecutive 16-byte chunks per instruction.
template <int CPR>
__device__ __forceinline__ int swz(int r, int c) {
    if constexpr (CPR == 8) return c ^ ((r & 7) ^ ((r >> 3) & 1));
    else return c ^ (r & 15);
}

// Element-type dependent pieces.
template <typename T, int D>
struct Ops;

// ------------------------------------------------------------------ bf16
template <int D>
struct Ops<__bf16, D> {
    static constexpr int kEsz = 2;
    static constexpr int kCPR = D / 8;         // 16-byte chunks per row
    static constexpr int kKRow = D;            // natural tile row stride (swizzled chunks)
    static constexpr int kVRow = kBC + 4;      // V^T row stride in LDS (elements)
    static constexpr int kKTile = kBC * kKRow; // elements per K tile
    static constexpr int kVTile = D * kVRow;   // elements per V^T tile
    static constexpr int kNS = D / 16;         // k-slices of a score block
    static constexpr int kChunks = kBC * D * kEsz / 16;  // 16-byte chunks per tile

    // Register-resident MFMA operand for NB blocks of 32 rows (the rows
    // that end up on the lanes of a score block).
    template <int NB = 2>
    struct QOp {
        bf16x8 q[NB][kNS];
    };

    // Operand rows R0 .. R0 + 32*NB - 1 of X (zero beyond L).
    template <int NB>
    __device__ __forceinline__ static void load_q(QOp<NB>& op, const __bf16* Xh, int R0, int L) {
        const int l = lane_id(), m = l & 31, h = l >> 5;
#pragma unroll
        for (int qb = 0; qb < NB; ++qb) {
            const int row = R0 + qb * 32 + m;
#pragma unroll
            for (int s = 0; s < kNS; ++s) {
                u32x4 v = {0u, 0u, 0u, 0u};
                if (row < L) v = *reinterpret_cast<const u32x4*>(Xh + (size_t)row * D + s * 16 + h * 8);
                op.q[qb][s] = __builtin_bit_cast(bf16x8, v);
            }
        }
    }

    // acc[kb][qb] = Tile[kb*32 + .., :] . Op[qb*32 + .., :]  (raw dot
    // products; tile rows in registers, operand rows on lanes)
    template <int NB>
    __device__ __forceinline__ static void scores(f32x16 (&acc)[2][NB], const __bf16* Kt, const QOp<NB>& op) {
        const int l = lane_id(), m = l & 31, h = l >> 5;
        if constexpr (NB == 1) {
            // one product per operand read: the next k-slice's operands are
            // read before this slice's products are issued, so that the LDS
            // latency overlaps the matrix core (the scheduler otherwise
            // waits on each read right before its product)
            auto rd = [&](int s, int kb) {
                const int row = kb * 32 + m;
                return __builtin_bit_cast(
                    bf16x8, *reinterpret_cast<const u32x4*>(Kt + row * kKRow + swz<kCPR>(row, 2 * s + h) * 8));
            };
            bf16x8 k[2][2];
            k[0][0] = rd(0, 0);
            k[0][1] = rd(0, 1);
            const f32x16 zero = {};
#pragma unroll
            for (int s = 0; s < kNS; ++s) {
                if (s + 1 < kNS) {
                    k[(s + 1) & 1][0] = rd(s + 1, 0);
                    k[(s + 1) & 1][1] = rd(s + 1, 1);
                }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
                    acc[kb][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k[s & 1][kb], op.q[0][s],
                                                                         s == 0 ? zero : acc[kb][0], 0, 0, 0);
                __builtin_amdgcn_sched_barrier(0);
            }
            return;
        }
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int qb = 0; qb < NB; ++qb)
#pragma unroll
                for (int i = 0; i < 16; ++i) acc[kb][qb][i] = 0.0f;
#pragma unroll
        for (int s = 0; s < kNS; ++s) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const int row = kb * 32 + m;
                const bf16x8 k = __builtin_bit_cast(
                    bf16x8, *reinterpret_cast<const u32x4*>(Kt + row * kKRow + swz<kCPR>(row, 2 * s + h) * 8));
#pragma unroll
                for (int qb = 0; qb < NB; ++qb)
                    acc[kb][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k, op.q[qb][s], acc[kb][qb], 0, 0, 0);
            }
        }
    }

    // Global -> registers: chunk c of the tile starting at key c0 (zero past
    // L; FULL: the caller knows the whole tile lies below L).
    template <bool FULL = false>
    __device__ __forceinline__ static u32x4 load_k_chunk(const __bf16* Kh, int c0, int L, int c) {
        const int key = c / (D / 8), ch = c % (D / 8);
        if (FULL) return *reinterpret_cast<const u32x4*>(Kh + (size_t)(c0 + key) * D + ch * 8);
        u32x4 v = {0u, 0u, 0u, 0u};
        if (c0 + key < L) v = *reinterpret_cast<const u32x4*>(Kh + (size_t)(c0 + key) * D + ch * 8);
        return v;
    }
    __device__ __forceinline__ static void store_k_chunk(__bf16* Kt, int c, u32x4 v) {
        const int key = c / (D / 8), ch = c % (D / 8);
        *reinterpret_cast<u32x4*>(Kt + key * kKRow + swz<kCPR>(key, ch) * 8) = v;
    }

    // V tile transposed into LDS: V^T[d][key].  Unit u covers 4 keys x 8 d.
    static constexpr int kVUnits = (kBC / 4) * (D / 8);
    struct VRegs {
        u32x4 r[4];
    };
    template <bool FULL = false>
    __device__ __forceinline__ static VRegs load_v_unit(const __bf16* Vh, int c0, int L, int u) {
        const int kg = u % (kBC / 4), dg = u / (kBC / 4);
        VRegs x;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int key = c0 + 4 * kg + i;
            if (FULL) {
                x.r[i] = *reinterpret_cast<const u32x4*>(Vh + (size_t)key * D + dg * 8);
            } else {
                u32x4 v = {0u, 0u, 0u, 0u};
                if (key < L) v = *reinterpret_cast<const u32x4*>(Vh + (size_t)key * D + dg * 8);
                x.r[i] = v;
            }
        }
        return x;
    }
    __device__ __forceinline__ static void store_v_unit(__bf16* Vt, int u, const VRegs& x) {
        const int kg = u % (kBC / 4), dg = u / (kBC / 4);
        // x.r[i] holds d = 8dg..8dg+7 of key 4kg+i; write 4 keys per d row.
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            uint32_t w[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) w[i] = (x.r[i][e >> 1] >> ((e & 1) * 16)) & 0xffffu;
            u32x2 pk;
            pk[0] = w[0] | (w[1] << 16);
            pk[1] = w[2] | (w[3] << 16);
            *reinterpret_cast<u32x2*>(Vt + (dg * 8 + e) * kVRow + 4 * kg) = pk;
        }
    }

    // The same transposed tile in fp16, each value times sc (a power of two
    // chosen so that the tile's largest magnitude stays below 2^15: then the
    // conversion is exact down to 2^-14, 29 binades below that maximum).
    __device__ __forceinline__ static void store_v_unit_f16(uint16_t* Vt, int u, const VRegs& x, float sc) {
        const int kg = u % (kBC / 4), dg = u / (kBC / 4);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            uint32_t w[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t bits = (x.r[i][e >> 1] >> ((e & 1) * 16)) & 0xffffu;
                w[i] = __builtin_bit_cast(uint16_t, (_Float16)(__builtin_bit_cast(float, bits << 16) * sc));
            }
            u32x2 pk;
            pk[0] = w[0] | (w[1] << 16);
            pk[1] = w[2] | (w[3] << 16);
            *reinterpret_cast<u32x2*>(Vt + (dg * 8 + e) * kVRow + 4 * kg) = pk;
        }
    }

    template <int NB = 2>
    struct OAcc {
        f32x16 o[D / 32][NB];
    };

    // The product below with the tile in fp16 (store_v_unit_f16) and the
    // weights times ws rounded to fp16: one MFMA per block instead of a
    // hi + lo pair.  ws must keep every |weight| * ws below 65504; rounding
    // to 11 bits errs by at most 2^-12 relative.
    template <int NB>
    __device__ __forceinline__ static void pv_f16(OAcc<NB>& oa, const uint16_t* Vt, const f32x16 (&a4)[2][NB],
                                                  const bool (&on)[2], float ws) {
        const int l = lane_id(), m = l & 31, h = l >> 5;
        if constexpr (NB == 1) {
            // products in (kb, t, db) order, each operand read one product
            // ahead (as in scores)
            constexpr int kDB = D / 32, kIt = 2 * 2 * kDB;
            auto rd = [&](int it) {
                const int kb = it / (2 * kDB), t = (it / kDB) & 1, db = it % kDB;
                const uint16_t* row = Vt + (db * 32 + m) * kVRow + kb * 32 + 16 * t + 4 * h;
                const u32x2 lo4 = *reinterpret_cast<const u32x2*>(row);
                const u32x2 hi4 = *reinterpret_cast<const u32x2*>(row + 8);
                u32x4 vv;
                vv[0] = lo4[0]; vv[1] = lo4[1]; vv[2] = hi4[0]; vv[3] = hi4[1];
                return __builtin_bit_cast(f16x8, vv);
            };
            f16x8 va[2], b;
            va[0] = rd(0);
#pragma unroll
            for (int it = 0; it < kIt; ++it) {
                const int kb = it / (2 * kDB), t = (it / kDB) & 1, db = it % kDB;
                if (db == 0) {
#pragma unroll
                    for (int p = 0; p < 8; ++p) b[p] = (_Float16)(a4[kb][0][8 * t + p] * ws);
                }
                if (it + 1 < kIt) va[(it + 1) & 1] = rd(it + 1);
                __builtin_amdgcn_sched_barrier(0);
                if (on[kb]) oa.o[db][0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(va[it & 1], b, oa.o[db][0], 0, 0, 0);
                __builtin_amdgcn_sched_barrier(0);
            }
            return;
        }
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            if (!on[kb]) continue;
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                f16x8 b[NB];
#pragma unroll
                for (int qb = 0; qb < NB; ++qb)
#pragma unroll
                    for (int p = 0; p < 8; ++p) b[qb][p] = (_Float16)(a4[kb][qb][8 * t + p] * ws);
#pragma unroll
                for (int db = 0; db < D / 32; ++db) {
                    const uint16_t* row = Vt + (db * 32 + m) * kVRow + kb * 32 + 16 * t + 4 * h;
                    const u32x2 lo4 = *reinterpret_cast<const u32x2*>(row);
                    const u32x2 hi4 = *reinterpret_cast<const u32x2*>(row + 8);
                    u32x4 vv;
                    vv[0] = lo4[0]; vv[1] = lo4[1]; vv[2] = hi4[0]; vv[3] = hi4[1];
                    const f16x8 va = __builtin_bit_cast(f16x8, vv);
#pragma unroll
                    for (int qb = 0; qb < NB; ++qb)
                        oa.o[db][qb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(va, b[qb], oa.o[db][qb], 0, 0, 0);
                }
            }
        }
    }

    // O^T[d][c] += Vt^T[d][tile rows of block kb] . W[rows][c] for the NB
    // operand blocks c: W arrives in score-block layout (tile rows in
    // registers, columns on lanes) and is split into bf16 hi + lo.  Vt is the
    // tile in PV layout (transposed, [d][row]).
    template <int NB>
    __device__ __forceinline__ static void pv(OAcc<NB>& oa, const __bf16* Vt, const f32x16 (&a4)[2][NB],
                                              const bool (&on)[2]) {
        const int l = lane_id(), m = l & 31, h = l >> 5;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            if (!on[kb]) continue;
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                bf16x8 bh[NB], bl[NB];
#pragma unroll
                for (int qb = 0; qb < NB; ++qb) {
#pragma unroll
                    for (int p = 0; p < 8; ++p) {
                        const float a = a4[kb][qb][8 * t + p];
                        const __bf16 hi = (__bf16)a;
                        bh[qb][p] = hi;
                        bl[qb][p] = (__bf16)(a - (float)hi);
                    }
                }
#pragma unroll
                for (int db = 0; db < D / 32; ++db) {
                    const __bf16* row = Vt + (db * 32 + m) * kVRow + kb * 32 + 16 * t + 4 * h;
                    const u32x2 lo4 = *reinterpret_cast<const u32x2*>(row);
                    const u32x2 hi4 = *reinterpret_cast<const u32x2*>(row + 8);
                    u32x4 vv;
                    vv[0] = lo4[0]; vv[1] = lo4[1]; vv[2] = hi4[0]; vv[3] = hi4[1];
                    const bf16x8 va = __builtin_bit_cast(bf16x8, vv);
#pragma unroll
                    for (int qb = 0; qb < NB; ++qb) {
                        oa.o[db][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, bh[qb], oa.o[db][qb], 0, 0, 0);
                        oa.o[db][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, bl[qb], oa.o[db][qb], 0, 0, 0);
                    }
                }
            }
        }
    }
};

// ------------------------------------------------------------------ fp32
template <int D>
struct Ops<float, D> {
    static constexpr int kEsz = 4;
    static constexpr int kCPR = D / 4;
    static constexpr int kKRow = D;
    static constexpr int kVRow = D + 4;          // V kept in natural [key][d] layout
    static constexpr int kKTile = kBC * kKRow;
    static constexpr int kVTile = kBC * kVRow;
    static constexpr int kChunks = kBC * D * kEsz / 16;

    template <int NB = 2>
    struct QOp {
        float q[NB][D / 2];
    };

    template <int NB>
    __device__ __forceinline__ static void load_q(QOp<NB>& op, const float* Xh, int R0, int L) {
        const int l = lane_id(), m = l & 31, h = l >> 5;
#pragma unroll
        for (int qb = 0; qb < NB; ++qb) {
            const int row = R0 + qb * 32 + m;
#pragma unroll
            for (int s = 0; s < D / 2; ++s) op.q[qb][s] = (row < L) ? Xh[(size_t)row * D + 2 * s + h] : 0.0f;
        }
    }

    template <int NB>
    __device__ __forceinline__ static void scores(f32x16 (&acc)[2][NB], const float* Kt, const QOp<NB>& op) {
        const int l = lane_id(), m = l & 31, h = l >> 5;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int qb = 0; qb < NB; ++qb)
#pragma unroll
                for (int i = 0; i < 16; ++i) acc[kb][qb][i] = 0.0f;
#pragma unroll
        for (int s = 0; s < D / 2; ++s) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const int row = kb * 32 + m, e = 2 * s + h;
                const float k = Kt[row * kKRow + swz<kCPR>(row, e >> 2) * 4 + (e & 3)];
#pragma unroll
                for (int qb = 0; qb < NB; ++qb)
                    acc[kb][qb] = __builtin_amdgcn_mfma_f32_32x32x2f32(k, op.q[qb][s], acc[kb][qb], 0, 0, 0);
            }
        }
    }

    template <bool FULL = false>
    __device__ __forceinline__ static u32x4 load_k_chunk(const float* Kh, int c0, int L, int c) {
        const int key = c / (D / 4), ch = c % (D / 4);
        if (FULL) return *reinterpret_cast<const u32x4*>(Kh + (size_t)(c0 + key) * D + ch * 4);
        u32x4 v = {0u, 0u, 0u, 0u};
        if (c0 + key < L) v = *reinterpret_cast<const u32x4*>(Kh + (size_t)(c0 + key) * D + ch * 4);
        return v;
    }
    __device__ __forceinline__ static void store_k_chunk(float* Kt, int c, u32x4 v) {
        const int key = c / (D / 4), ch = c % (D / 4);
        *reinterpret_cast<u32x4*>(Kt + key * kKRow + swz<kCPR>(key, ch) * 4) = v;
    }

    // V stays in natural layout: a unit is one 16-byte chunk.
    static constexpr int kVUnits = kChunks;
    struct VRegs {
        u32x4 r;
    };
    template <bool FULL = false>
    __device__ __forceinline__ static VRegs load_v_unit(const float* Vh, int c0, int L, int u) {
        VRegs x;
        x.r = load_k_chunk<FULL>(Vh, c0, L, u);
        return x;
    }
    __device__ __forceinline__ static void store_v_unit(float* Vt, int u, const VRegs& x) {
        const int key = u / (D / 4), ch = u % (D / 4);
        *reinterpret_cast<u32x4*>(Vt + key * kVRow + ch * 4) = x.r;
    }

    template <int NB = 2>
    struct OAcc {
        f32x16 o[D / 32][NB];
    };

    // fp32: the PV layout is the natural [row][d] layout.
    template <int NB>
    __device__ __forceinline__ static void pv(OAcc<NB>& oa, const float* Vt, const f32x16 (&a4)[2][NB],
                                              const bool (&on)[2]) {
        const int l = lane_id(), m = l & 31, h = l >> 5;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            if (!on[kb]) continue;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = kb * 32 + key_of_reg(r, h);
#pragma unroll
                for (int db = 0; db < D / 32; ++db) {
                    const float va = Vt[key * kVRow + db * 32 + m];
#pragma unroll
                    for (int qb = 0; qb < NB; ++qb)
                        oa.o[db][qb] = __builtin_amdgcn_mfma_f32_32x32x2f32(va, a4[kb][qb][r], oa.o[db][qb], 0, 0, 0);
                }
            }
        }
    }
};

// Set masked elements of a partial tile to -inf.  Register r of lane half h
// holds key jb + c(r) of the lane's query, c(r) = 8 (r / 4) + r % 4 a
// compile-time offset, so every condition of key_active reduces to one
// interval lo <= c(r) <= hi per lane and 32-key block (plus key 0 under the
// sink): two compares with constants and a select per element.
template <int NB>
__device__ __forceinline__ void apply_mask(f32x16 (&acc)[2][NB], int J, int R0, const Geom& g) {
    const int l = lane_id(), m = l & 31, h = l >> 5;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
        const int jb = J * kBC + kb * 32 + 4 * h;
        const bool sink = (g.mode == 2) & (jb == 0);
#pragma unroll
        for (int qb = 0; qb < NB; ++qb) {
            const int i = R0 + qb * 32 + m;
            int hi = g.L - 1 - jb;                        // key < L
            if (g.mode >= 1) hi = min(hi, i - jb);        // key <= query
            if (i >= g.L) hi = -1;                        // query < L
            const int lo = (g.mode == 2) ? i - jb - g.W : INT_MIN;  // query - key <= W
            f32x16 a = acc[kb][qb];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int c = 8 * (r >> 2) + (r & 3);
                const bool act = (c <= hi) & ((c >= lo) | ((r == 0) & sink));
                a[r] = act ? a[r] : neg_inf();
            }
            acc[kb][qb] = a;
        }
    }
}

// Class of the block rows [i0, i0 + ni) x keys [c0, c0 + nc) under the mask.
__device__ __forceinline__ int block_class(int i0, int ni, int c0, int nc, const Geom& g) {
    const int i1 = i0 + ni - 1, c1 = c0 + nc - 1;
    if (c0 >= g.L || i0 >= g.L) return kSkip;
    if (g.mode >= 1 && c0 > i1) return kSkip;
    if (g.mode == 2 && c0 != 0 && i0 - c1 > g.W) return kSkip;
    bool full = (c1 < g.L) && (i1 < g.L);
    if (g.mode >= 1) full = full && (c1 <= i0);
    if (g.mode == 2) full = full && (i1 - c0 <= g.W);
    return full ? kFull : kPartial;
}

// Masking for score blocks whose tile rows (registers) are QUERIES and whose
// lanes are KEYS (the backward's dK/dV orientation): register r of lane half
// h holds query ib + c(r), so the conditions again reduce to one interval of
// c(r) per lane (the sink column, key 0, drops the window bound).
template <int NB>
__device__ __forceinline__ void apply_mask_rows_are_queries(f32x16 (&acc)[2][NB], int I0, int C0, const Geom& g) {
    const int l = lane_id(), m = l & 31, h = l >> 5;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
        const int ib = I0 + kb * 32 + 4 * h;
#pragma unroll
        for (int cb = 0; cb < NB; ++cb) {
            const int j = C0 + cb * 32 + m;
            int hi = g.L - 1 - ib;                                       // query < L
            if ((g.mode == 2) & (j != 0)) hi = min(hi, j - ib + g.W);    // query - key <= W
            if (j >= g.L) hi = -1;                                       // key < L
            const int lo = (g.mode >= 1) ? j - ib : INT_MIN;             // key <= query
            f32x16 a = acc[kb][cb];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int c = 8 * (r >> 2) + (r & 3);
                a[r] = ((c <= hi) & (c >= lo)) ? a[r] : neg_inf();
            }
            acc[kb][cb] = a;
        }
    }
}

// Work item -> (bh, first row).  Items of one q-block rank are consecutive
// across heads, so the 8 XCDs (blocks dealt round-robin) each see a few
// heads; causal runs take the longest rows first.
__device__ __forceinline__ void decode_item(int item, int BH, int nQ, bool heavy_first, int& bh, int& r0) {
    bh = item % BH;
    const int qi = item / BH;
    r0 = (heavy_first ? (nQ - 1 - qi) : qi) * kBR;
}

}  // namespace attn
}  // namespace entmax
