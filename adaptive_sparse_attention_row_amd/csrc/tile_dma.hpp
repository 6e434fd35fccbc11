// tile_dma.hpp -- direct global -> LDS staging of 64-row tiles (gfx950
// global_load_lds_dwordx4) into a ring of stages, with explicit counter waits.
//
// Each DMA instruction writes the 16 bytes of each of the 64 lanes to 64
// consecutive 16-byte LDS slots starting at a wave-uniform base; the global
// address of each lane is free.  A tile's slot (row r, position p) is filled
// from chunk swz(r, p) of that row, which produces the swizzled natural
// layout the score reads expect (swz is its own inverse).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_common.hpp"

namespace entmax {
namespace attn {

// s_waitcnt with vmcnt <= N and no wait on the other counters (gfx9 encoding:
// vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier that first drains this wave's LDS operations but leaves
// outstanding global loads (the prefetch ring) in flight.
__device__ __forceinline__ void barrier_keep_vm() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4) | (0 << 8));  // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

template <typename T, int D>
struct TileDMA {
    static constexpr int kCPR = D * (int)sizeof(T) / 16;  // 16-byte chunks per row
    static constexpr int kTileCh = 64 * kCPR;             // chunks per tile
    static constexpr int kTileElems = 64 * D;

    // Number of DMA instructions each thread issues for NT tiles.
    template <int NT>
    static constexpr int instrs() {
        return NT * kTileCh / kNT;
    }

    // Per-lane parts of the DMA addresses, fixed for a kernel: for each of a
    // thread's instructions, the row within its tile, the tile index (the
    // same for the whole wave), the element offset of the (swizzled) source
    // chunk within that row, and row and chunk together as one offset from
    // the tile's first element.
    template <int NT>
    struct Lanes {
        static constexpr int kIpw = NT * kTileCh / 4 / kWave;
        int row[kIpw];
        int tile[kIpw];
        int col[kIpw];
        int off[kIpw];
    };

    template <int NT>
    __device__ __forceinline__ static Lanes<NT> lanes() {
        const int t = threadIdx.x, lane = t & (kWave - 1);
        const int w = wave_id();
        constexpr int kPerWave = NT * kTileCh / 4;
        Lanes<NT> ln;
#pragma unroll
        for (int k = 0; k < Lanes<NT>::kIpw; ++k) {
            const int q = w * kPerWave + k * kWave + lane;
            const int qt = q % kTileCh;
            ln.tile[k] = __builtin_amdgcn_readfirstlane(q / kTileCh);
            ln.row[k] = qt / kCPR;
            ln.col[k] = swz<kCPR>(ln.row[k], qt % kCPR) * (16 / (int)sizeof(T));
            ln.off[k] = ln.row[k] * D + ln.col[k];
        }
        return ln;
    }

    // Stage NT tiles (rows r0[k] .. r0[k] + 63 of X; rows past L read row
    // L - 1, junk that the masks discard) into dst (NT tiles back to back).
    // r0 must be wave-uniform: a tile inside [0, L) is then addressed from a
    // scalar base plus the lane's fixed offset.
    template <int NT>
    __device__ __forceinline__ static void issue(T* dst, const T* Xh, const int (&r0)[NT], int L,
                                                 const Lanes<NT>& ln) {
        const int w = wave_id();
        constexpr int kPerWave = NT * kTileCh / 4;
        constexpr int kIpw = Lanes<NT>::kIpw;
        static_assert(kIpw * kWave * 4 == NT * kTileCh, "tile chunks must split evenly");
        int rmax = r0[0];
#pragma unroll
        for (int k = 1; k < NT; ++k) rmax = rmax > r0[k] ? rmax : r0[k];
        // (with more than four instructions per thread the offset table costs
        // more registers than it saves instructions: rows are recomputed)
        if (kIpw <= 4 && rmax + 64 <= L) {
#pragma unroll
            for (int k = 0; k < kIpw; ++k) {
                const int q0 = w * kPerWave + k * kWave;  // first slot of this instruction
                const T* tb = Xh + (size_t)r0[ln.tile[k]] * D;
                T* base = dst + q0 * (16 / (int)sizeof(T));
                __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(tb + (uint32_t)ln.off[k]),
                                                 (__attribute__((address_space(3))) void*)(base), 16, 0, 0);
            }
        } else {
#pragma unroll
            for (int k = 0; k < kIpw; ++k) {
                const int q0 = w * kPerWave + k * kWave;
                int row = r0[ln.tile[k]] + ln.row[k];
                if (rmax + 64 > L) row = row < L ? row : L - 1;
                const T* src = Xh + (size_t)row * D + ln.col[k];
                T* base = dst + q0 * (16 / (int)sizeof(T));
                __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(src),
                                                 (__attribute__((address_space(3))) void*)(base), 16, 0, 0);
            }
        }
    }
};

}  // namespace attn
}  // namespace entmax
