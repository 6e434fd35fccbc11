// attn_fwd.hip -- 1.5-entmax attention forward on gfx950.
//
// One workgroup per 128 query rows of a head runs three phases:
//
// stats   one sweep over the tiles the mask mode allows: S^T = K Q^T on
//         MFMA; per row the maximum and the sixteen largest tile maxima
//         (four per lane half and key parity); per (row half, tile) the
//         largest score.  tau_lo = the exact threshold of those tile
//         maxima.  Adding scores to a row only raises its threshold (every
//         term of the normaliser is non-negative), so tau_lo <= tau, and
//         it also clears the bracket end max - 2 of "AdaSplash-2: Faster
//         Differentiable Sparse Attention" sec. 2.4 (score units).
// solve   collect: over the tiles whose largest score beats tau_lo, every
//         score s > tau_lo is appended to its row's candidate sub-list of
//         the sweeping lane (no atomics: the lists and every sum over them
//         are the same on every call).  Nothing at or below tau_lo can carry
//         weight, so the row's threshold is the threshold of its candidates.
//         solve: per row, Newton steps from below on the candidates
//         (f(t) = sum [(s - t)/2]_+^2 - 1 is convex and decreasing) with a
//         bisection guard and an exact finish: once tau lies below the
//         support the normaliser is a quadratic in tau over {s > tau}
//         (S0/S1/S2 of AdaSplash-2 appendix C.3).  Sums are fp64.
//         mask: a 64x64 tile is non-null iff one of its candidates exceeds
//         its row's tau (packed 32 tiles per word, AdaSplash-2 appendix C.4).
//         overflow: rows whose lists overflow take the histogram
//         initialisation of AdaSplash-2 sec. 3.1 (left-edge bins, exact
//         solve on the bin counts), are collected again above tau_h when
//         that fits, else refined by Halley-bisection sweeps on the
//         histogram bracket.
// out     O: from the candidate lists (the support's V rows) when they are
//         short next to the non-null tiles; otherwise by walking only the set
//         mask bits (find-first-set over the packed words, AdaSplash-2
//         sec. 3.3 phase 4), recomputing S and A = [(S - tau)/2]_+^2 and
//         accumulating O = A V on MFMA.  For bf16 inputs the product takes A
//         and V in fp16 (A <= 1 keeps 11 significant bits, and bf16 V
//         converts exactly while |V| <= 65504; a bf16 A alone measured
//         6.6e-3 error against the 2e-3 bound), with a bf16 hi + lo redo of
//         a block whose V leaves the fp16 range.
//
// For bf16 inputs with L <= 16384 the three phases run in one fused kernel
// (fwd_fused_kernel) whose row statistics, tile maxima, tile lists and mask
// stay in LDS between the phases.  fp32 inputs, longer sequences and the
// phase entry points (entmax_attn_score_stats, entmax_attn_output) launch
// each phase as its own kernel (fwd_stats_kernel, fwd_solve_kernel,
// fwd_out_kernel / fwd_out_bf16_kernel), passing state through the
// workspace.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_common.hpp"
#include "device_common.hpp"
#include "launch.hpp"
#include "tile_dma.hpp"

namespace entmax {
namespace attn {
namespace {

constexpr int kMaxIter = 40;   // solver iterations
constexpr int kFbMaxIter = 60; // fallback sweeps

struct FwdParams {
    const void* q;
    const void* k;
    const void* v;
    float* o;
    float* tau;
    uint32_t* mask;   // [BH][Tr64][Wd]
    float* rowstat;   // workspace [BH][L][2]: row max, tau_lo (score units)
    float* umax;      // workspace [BH][Tr64][Tc]: largest raw score per (64-row block, tile)
    u32x2* clist;     // workspace [BH * nQ][kCandCap][128]: candidates (score bits, key index), slot-major per row block
    int* ostate;      // workspace [BH * nQ]: 1 where the solve kernel wrote O itself (null: the output kernel writes all)
    float* gv;        // [BH][L][d]: sum_j g_ij V_j, g = dA/dS (null: not requested; fused kernel only)
    float* gsum;      // [BH][L]: sum_j g_ij
    int gather;       // the solve kernel writes O from the candidate lists where it can
    int BH, L, mode, W, nQ, Tc, Tr64, Wd;
    float scale;
    int cap;
    AlphaMap am;  // the alpha-entmax map
    int gen;      // alpha != 1.5: Newton solves and pow weights
};

// Candidate slots per row (all four sub-lists, LDS and workspace).
constexpr int kCandCap = 128;

// ------------------------------------------------------------ tile lists
// Build a list of tile indices with per-row-half flags (bit 0: qh 0,
// bit 1: qh 1), entries J | flags << 12, in increasing J.  One wave builds;
// flags_of(J) is evaluated per lane.
template <class FlagsOf>
__device__ __forceinline__ int build_list(uint16_t* list, int Tc, FlagsOf flags_of) {
    const int l = lane_id();
    int n = 0;
    for (int base = 0; base < Tc; base += kWave) {
        const int J = base + l;
        const int f = (J < Tc) ? flags_of(J) : 0;
        const uint64_t b = __ballot(f != 0);
        if (f) list[n + lanes_below(b)] = (uint16_t)(J | (f << 12));
        n += __popcll(b);
    }
    return n;
}

// ------------------------------------------------------------ sweeps
// Stream the tiles of `list` in pairs (wave kh takes entry 2p + kh), staging
// K (and V when WITH_V) through LDS, and call fn(J, cls, acc) for every tile
// flagged for this wave's row half.
template <typename T, int D, int NBUF, bool WITH_V, class Fn>
__device__ __forceinline__ void sweep(const uint16_t* list, int n, const T* Kh, const T* Vh, T* kbuf, T* vbuf,
                      const typename Ops<T, D>::template QOp<2>& qop, int R0, const Geom& g, Fn fn) {
    using O = Ops<T, D>;
    const int t = threadIdx.x, w = wave_id(), qh = w & 1, kh = w >> 1;
    constexpr int kKPer = 2 * O::kChunks / kNT;                         // K chunks per thread per pair
    constexpr int kVPer = WITH_V ? (2 * O::kVUnits + kNT - 1) / kNT : 0;  // V units per thread per pair
    const int npairs = (n + 1) / 2;
    if (npairs == 0) return;

    u32x4 kr[kKPer];
    typename O::VRegs vr[kVPer > 0 ? kVPer : 1];

    auto load = [&](int p) {
#pragma unroll
        for (int i = 0; i < kKPer; ++i) {
            const int c = t + kNT * i;
            const int sel = c / O::kChunks, cc = c % O::kChunks;
            const int e = 2 * p + sel;
            const int J = (e < n) ? (list[e] & 0xfff) : 0;
            const int c0 = (e < n) ? J * kBC : g.L;  // past L: zeros
            kr[i] = O::load_k_chunk(Kh, c0, g.L, cc);
        }
        if constexpr (WITH_V) {
#pragma unroll
            for (int i = 0; i < kVPer; ++i) {
                const int u = t + kNT * i;
                if (u < 2 * O::kVUnits) {
                    const int sel = u / O::kVUnits, uu = u % O::kVUnits;
                    const int e = 2 * p + sel;
                    const int J = (e < n) ? (list[e] & 0xfff) : 0;
                    const int c0 = (e < n) ? J * kBC : g.L;
                    vr[i] = O::load_v_unit(Vh, c0, g.L, uu);
                }
            }
        }
    };
    auto store = [&](int buf) {
#pragma unroll
        for (int i = 0; i < kKPer; ++i) {
            const int c = t + kNT * i;
            const int sel = c / O::kChunks, cc = c % O::kChunks;
            O::store_k_chunk(kbuf + (buf * 2 + sel) * O::kKTile, cc, kr[i]);
        }
        if constexpr (WITH_V) {
#pragma unroll
            for (int i = 0; i < kVPer; ++i) {
                const int u = t + kNT * i;
                if (u < 2 * O::kVUnits) {
                    const int sel = u / O::kVUnits, uu = u % O::kVUnits;
                    O::store_v_unit(vbuf + (buf * 2 + sel) * O::kVTile, uu, vr[i]);
                }
            }
        }
    };

    load(0);
    store(0);
    for (int p = 0; p < npairs; ++p) {
        const int buf = (NBUF == 2) ? (p & 1) : 0;
        __syncthreads();
        if (NBUF == 2 && p + 1 < npairs) load(p + 1);
        const int e = 2 * p + kh;
        if (e < n) {
            const int ent = list[e];
            const int J = ent & 0xfff;
            if ((ent >> (12 + qh)) & 1) {
                const int cls = tile_class(J, R0, g);
                if (cls != kSkip) {
                    f32x16 acc[2][2];
                    O::scores(acc, kbuf + (buf * 2 + kh) * O::kKTile, qop);
                    if (cls == kPartial) apply_mask(acc, J, R0, g);
                    fn(J, cls, acc, WITH_V ? vbuf + (buf * 2 + kh) * O::kVTile : nullptr);
                }
            }
        }
        if (p + 1 < npairs) {
            if (NBUF == 2) {
                store(buf ^ 1);
            } else {
                __syncthreads();
                load(p + 1);
                store(0);
            }
        }
    }
    __syncthreads();
}

// --------------------------------------------------------- DMA ring sweep
// Stream the tiles of `list` in pairs (wave kh takes entry 2p + kh) through
// an S-stage ring filled by direct global->LDS loads, keeping S - 1 pairs in
// flight, and call fn(J, e, acc) for every tile flagged for this wave's row
// half (e: the tile's position in the list).  One barrier per pair; the
// global loads stay outstanding across it.  (The compiler makes the first LDS
// read after a direct load wait for all loads in flight; reading a stage
// before issuing the next loads, or hiding the reads from it, measured no
// faster here, so the plain order stays.)
template <typename T, int D, int S, class Fn>
__device__ __forceinline__ void ring_sweep(const uint16_t* list, int n, const T* Kh, T* ring,
                                           const typename Ops<T, D>::template QOp<2>& qop, int R0,
                                           const Geom& g, Fn fn) {
    using O = Ops<T, D>;
    using DMA = TileDMA<T, D>;
    constexpr int kIpp = DMA::template instrs<2>();
    constexpr int kStage = 2 * DMA::kTileElems;
    const int w = wave_id(), qh = w & 1, kh = w >> 1;
    const int npairs = (n + 1) / 2;
    if (npairs == 0) return;
    const auto ln = DMA::template lanes<2>();
    // list entries are the same for the whole wave: read them into scalars
    auto issue = [&](int pp) {
        int r0[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int e = 2 * pp + u;
            r0[u] = (e < n) ? (__builtin_amdgcn_readfirstlane(list[e]) & 0xfff) * kBC : 0;
        }
        DMA::template issue<2>(ring + (pp % S) * kStage, Kh, r0, g.L, ln);
    };
    // this wave's tile of pair pp: list entry, key tile, mask class (kSkip: none)
    auto tile_of = [&](int pp, int& e, int& J) -> int {
        e = 2 * pp + kh;
        if (e >= n) return kSkip;
        const int ent = __builtin_amdgcn_readfirstlane(list[e]);
        J = ent & 0xfff;
        if (!((ent >> (12 + qh)) & 1)) return kSkip;
        return tile_class(J, R0, g);
    };
    // S-stage ring keeping S - 1 pairs in flight (S == 1: load, then use)
#pragma unroll
    for (int pp = 0; pp < S - 1; ++pp)
        if (pp < npairs) issue(pp);
    for (int pp = 0; pp < npairs; ++pp) {
        if constexpr (S == 1) {
            barrier_keep_vm();
            issue(pp);
            wait_vmcnt<0>();
        } else {
            if (npairs - 1 - pp >= S - 2) wait_vmcnt<(S - 2) * kIpp>();
            else wait_vmcnt<0>();
        }
        barrier_keep_vm();
        if (S > 1 && pp + S - 1 < npairs) issue(pp + S - 1);
        int e = 0, J = 0;
        const int cls = tile_of(pp, e, J);
        if (cls != kSkip) {
            const T* Kt = ring + (pp % S) * kStage + kh * DMA::kTileElems;
            f32x16 acc[2][2];
            O::scores(acc, Kt, qop);
            if (cls == kPartial) apply_mask(acc, J, R0, g);
            fn(J, e, acc);
        }
    }
    __syncthreads();
}

// The same sweep for a workgroup whose tiles are the first nt key tiles:
// no mask (nt = all tiles) or the causal mask (nt = up to the diagonal), with
// every key tile inside L (L a multiple of 64) and all 128 query rows below
// L.  Pair pp is then tiles 2 pp and 2 pp + 1, so no list is read, a tile
// class is evaluated only on the diagonal, and each wave stages the same
// half of one tile of every pair from a scalar tile base plus per-lane byte
// offsets computed once: per pair, what is left besides the products and
// the statistics is the DMA issue, one wait and the barrier.
template <typename T, int D, int S, bool CAUSAL, class Fn>
__device__ __forceinline__ void dense_sweep(int nt, const T* Kh, T* ring,
                                            const typename Ops<T, D>::template QOp<2>& qop, int R0,
                                            const Geom& g, Fn fn) {
    using O = Ops<T, D>;
    using DMA = TileDMA<T, D>;
    static_assert(S >= 2, "the dense sweep keeps at least one pair in flight");
    constexpr int kIpw = DMA::template Lanes<2>::kIpw;  // DMA instructions per thread per pair
    constexpr int kPerWave = DMA::kTileCh / 2;           // 16-byte slots per wave per pair
    constexpr int kStage = 2 * DMA::kTileElems;
    constexpr int kSlotElems = 16 / (int)sizeof(T);
    constexpr size_t kTileBytes = (size_t)64 * D * sizeof(T);
    const int w = wave_id(), kh = w >> 1, lane = lane_id();
    const int npairs = (nt + 1) / 2;
    uint32_t off[kIpw];
#pragma unroll
    for (int k = 0; k < kIpw; ++k) {
        const int qt = (w * kPerWave + k * kWave + lane) % DMA::kTileCh;
        const int row = qt / DMA::kCPR;
        off[k] = (uint32_t)((row * D + swz<DMA::kCPR>(row, qt % DMA::kCPR) * kSlotElems) * sizeof(T));
    }
    // wave w stages half (w & 1) of tile (w >> 1) of each pair; the second
    // tile of a last, odd pair lies past the range, and its waves re-read the
    // first (the products skip it)
    const char* kw = reinterpret_cast<const char*>(Kh) + (size_t)(w >> 1) * kTileBytes;
    auto issue = [&](int pq, int stage) {
        const char* tb = CAUSAL ? reinterpret_cast<const char*>(Kh) + (size_t)min(2 * pq + (w >> 1), nt - 1) * kTileBytes
                                : kw + (size_t)pq * 2 * kTileBytes;
        T* base = ring + stage * kStage + w * kPerWave * kSlotElems;
#pragma unroll
        for (int k = 0; k < kIpw; ++k)
            __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(tb + off[k]),
                                             (__attribute__((address_space(3))) void*)(base + k * kWave * kSlotElems),
                                             16, 0, 0);
    };
#pragma unroll
    for (int pp = 0; pp < S - 1; ++pp)
        if (pp < npairs) issue(pp, pp);
    int su = 0, si = S - 1;  // stage read this pair, stage the next issue fills
    for (int pp = 0; pp < npairs; ++pp) {
        if (npairs - 1 - pp >= S - 2) wait_vmcnt<(S - 2) * kIpw>();
        else wait_vmcnt<0>();
        barrier_keep_vm();
        if (pp + S - 1 < npairs) issue(pp + S - 1, si);
        const int J = 2 * pp + kh;
        if constexpr (CAUSAL) {
            // only the diagonal tiles are partial or empty
            const int cls = J >= nt ? kSkip : (J * kBC + kBC - 1 <= R0) ? kFull : tile_class(J, R0, g);
            if (cls != kSkip) {
                f32x16 acc[2][2];
                O::scores(acc, ring + su * kStage + kh * DMA::kTileElems, qop);
                if (cls == kPartial) apply_mask(acc, J, R0, g);
                fn(J, J, acc);
            }
        } else {
            f32x16 acc[2][2];
            O::scores(acc, ring + su * kStage + kh * DMA::kTileElems, qop);
            fn(J, J, acc);
        }
        su = su + 1 == S ? 0 : su + 1;
        si = si + 1 == S ? 0 : si + 1;
    }
    __syncthreads();
}

// Maximum over the 64 lanes of a wave, by DPP row shifts and broadcasts
// (VALU only), returned to every lane.  Each step is one v_max_f32 with a
// DPP source; a lane without a source is not written and keeps its value,
// which is what the max would give.  (The compiler does not fold a DPP move
// whose fallback value is live into its user, hence the assembly; the
// s_nop covers the two wait states a DPP read of a VGPR written by the
// previous VALU instruction needs.)
#define ENTMAX_DPP_MAX(ctrl)                                                       \
    asm("s_nop 1\n\tv_max_f32_dpp %0, %1, %1 " ctrl " bank_mask:0xf" : "=v"(y) : "v"(x), "0"(x)); \
    x = y
__device__ __forceinline__ float wave_max_dpp(float x) {
    float y;
    ENTMAX_DPP_MAX("row_shr:1 row_mask:0xf");
    ENTMAX_DPP_MAX("row_shr:2 row_mask:0xf");
    ENTMAX_DPP_MAX("row_shr:4 row_mask:0xf");
    ENTMAX_DPP_MAX("row_shr:8 row_mask:0xf");     // lane 15 of each row holds the row max
    ENTMAX_DPP_MAX("row_bcast:15 row_mask:0xa");
    ENTMAX_DPP_MAX("row_bcast:31 row_mask:0xc");  // lane 63 holds the wave max
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 63));
}
#undef ENTMAX_DPP_MAX

// --------------------------------------------------------- small solvers
// Exact threshold of N sorted-descending values (score units, -inf entries
// absent): scan of the top-k prefixes, each a quadratic in tau.
template <int N>
__device__ __forceinline__ float tau_of_sorted(const float (&x)[N]) {
    const float m = x[0];
    float a = 0.f, b = 0.f, best = -2.0f;
#pragma unroll
    for (int k = 1; k <= N; ++k) {
        const float xv = x[k - 1];
        const bool live = xv > neg_inf();
        const float y = live ? xv - m : 0.f;
        a += y;
        b += y * y;
        const float disc = a * a - (float)k * (b - 4.0f);
        const float tk = (a - sqrtf(fmaxf(disc, 0.f))) / (float)k;
        if (live && disc >= 0.f && tk <= y) best = tk;
    }
    return m + best;
}

// General alpha: a lower bound on the threshold of N values (-inf entries
// absent): Newton from below from the bracket end max - 1/(alpha-1); the last
// point with f >= 0, less a margin for the rounding of its sums.
template <int N>
__device__ __forceinline__ float tau_lower_gen(const float (&x)[N], const AlphaMap& am) {
    float m = neg_inf(), n = 0.f;
#pragma unroll
    for (int k = 0; k < N; ++k) {
        m = fmaxf(m, x[k]);
        n += x[k] > neg_inf() ? 1.f : 0.f;
    }
    float lo = m - am.e, hi = am.hi(m, n), t = lo;
    for (int it = 0; it < 30; ++it) {
        float F = 0.f, F1 = 0.f;
#pragma unroll
        for (int k = 0; k < N; ++k) {
            const float u = am.am1 * (x[k] - t);
            if (u > 0.f) {
                const float q = am.pw1(u);  // p / u
                F = fmaf(q, u, F);
                F1 += q;
            }
        }
        bool fin;
        const float tn = newton_or_bisect(t, F, F1, lo, hi, &fin, am);
        if (fin || hi - lo <= 4e-7f * fmaxf(1.0f, fabsf(t))) break;
        t = tn;
    }
    return lo - 1e-6f * fmaxf(1.0f, fabsf(lo));
}

// Sort N (a power of two) values descending in registers (bitonic network).
template <int N>
__device__ __forceinline__ void sort_desc(float (&x)[N]) {
#pragma unroll
    for (int k = 2; k <= N; k <<= 1)
#pragma unroll
        for (int j = k >> 1; j > 0; j >>= 1)
#pragma unroll
            for (int i = 0; i < N; ++i) {
                const int l = i ^ j;
                if (l > i) {
                    const bool desc = (i & k) == 0;
                    const float a = x[i], b = x[l];
                    const float hi = fmaxf(a, b), lo = fminf(a, b);
                    x[i] = desc ? hi : lo;
                    x[l] = desc ? lo : hi;
                }
            }
}

// ------------------------------------------------------------ candidate lists
// A row's candidates live in four sub-lists, one for each (key-parity wave
// kh, lane half h) that sweeps the row: entry c of sub-list q = 2 kh + h
// sits in slot 4c + q of the workspace, slot-major over the 128 rows of the
// workgroup, as (score bits, key index within the head).  Each sub-list is
// written by one lane only, in the order that lane meets its scores (tile-list
// order, then register order): no atomics, and the lists -- and every sum
// taken over them in list order -- are the same on every call.
constexpr int kCapQ = kCandCap / 4;     // entries per sub-list

// The entries read by lane half h of the pair of lanes that solves a row:
// sub-list h (wave kh = 0), then sub-list 2 + h (wave kh = 1).
struct CandSrc {
    const u32x2* glob;  // clist + row
    int n0, n1;         // entries of the two sub-lists
    int h;
    __device__ __forceinline__ int n() const { return n0 + n1; }
    __device__ __forceinline__ int slot(int i) const { return i < n0 ? 4 * i + h : 4 * (i - n0) + 2 + h; }
    __device__ __forceinline__ u32x2 entry(int i) const { return glob[(size_t)slot(i) * kBR]; }
    __device__ __forceinline__ float at(int i) const { return __builtin_bit_cast(float, entry(i)[0]); }
    // f(x) for entries i0, i0 + 1, ... in order.  Four entries per step are
    // loaded at once from clamped slots (every slot of i in [0, n) lies inside
    // the lists); entries past a lane's list read -inf, which every caller's
    // f ignores (no threshold test passes).  The step count is wave-uniform.
    template <class F>
    __device__ __forceinline__ void each_from(int i0, F f) const {
        const int n = n0 + n1;
        for (int k = i0; __builtin_amdgcn_ballot_w64(k < n) != 0; k += 4) {
            float x[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int i = k + u;
                const float y = at(max(min(i, n - 1), 0));
                x[u] = (i < n) ? y : neg_inf();
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) f(x[u]);
        }
    }
    template <class F>
    __device__ __forceinline__ void each(F f) const { each_from(0, f); }
};

// The same entries: the first KR scores in registers (missing entries read
// -inf, which no threshold test passes), their keys and the next KL scores
// in a column of LDS that only this thread touches (col[k * kNT]: keys for
// k < KR, scores for KR <= k < KR + KL), any further ones read from the
// workspace on each pass.  Every pass visits the entries in list order.  The
// slots of the first KR + KL entries lie inside the block's lists (slot(i) <
// 4 (KR + KL) <= kCandCap), so they are loaded unconditionally, all at once.
template <int KR, int KL>
struct RegSrc {
    static_assert(4 * (KR + KL) <= kCandCap, "entries' slots inside the lists");
    float v[KR];
    CandSrc src;
    uint32_t* col;
    int nl;
    __device__ __forceinline__ void load(const CandSrc& s, uint32_t* lds_col) {
        src = s;
        col = lds_col;
        const int n = s.n();
        // (the LDS scores only in waves where some lane's list is longer than
        // the registers: a wave-uniform branch)
        const bool longer = __builtin_amdgcn_ballot_w64(n > KR) != 0;
        u32x2 e[KR];
        uint32_t x[KL > 0 ? KL : 1];
#pragma unroll
        for (int k = 0; k < KR; ++k) e[k] = s.entry(k);
        if (longer) {
#pragma unroll
            for (int k = 0; k < KL; ++k) x[k] = __builtin_bit_cast(uint32_t, s.at(KR + k));
        }
#pragma unroll
        for (int k = 0; k < KR; ++k) {
            v[k] = (k < n) ? __builtin_bit_cast(float, e[k][0]) : neg_inf();
            col[k * kNT] = e[k][1];
        }
        if (longer) {
#pragma unroll
            for (int k = 0; k < KL; ++k) col[(KR + k) * kNT] = x[k];
        }
        nl = min(max(n - KR, 0), KL);
    }
    __device__ __forceinline__ uint32_t key(int k) const { return col[k * kNT]; }
    template <class F>
    __device__ __forceinline__ void each(F f) const {
#pragma unroll
        for (int k = 0; k < KR; ++k) f(v[k]);
        for (int k = 0; k < nl; ++k) f(__builtin_bit_cast(float, col[(KR + k) * kNT]));
        src.each_from(KR + nl, f);
    }
};

// The raw dot-product threshold equivalent to a score threshold: x > raw
// exactly when fl(x * scale) > lo (fl(x * scale) is non-decreasing in x),
// so the sweeps compare raw products and scale only what they keep.
__device__ __forceinline__ float next_up(float x) {
    if (x == __builtin_inff() || x != x) return x;
    if (x == 0.0f) return __builtin_bit_cast(float, 1u);
    const uint32_t b = __builtin_bit_cast(uint32_t, x);
    return __builtin_bit_cast(float, x > 0.0f ? b + 1u : b - 1u);
}
__device__ __forceinline__ float next_down(float x) { return -next_up(-x); }
__device__ __forceinline__ float raw_threshold(float lo, float scale) {
    if (!(lo > neg_inf()) || !(lo < __builtin_inff())) return lo;
    float r = lo / scale;
    for (int i = 0; i < 4 && r * scale > lo; ++i) r = next_down(r);
    for (int i = 0; i < 4 && next_up(r) * scale <= lo; ++i) r = next_up(r);
    return r;
}

// Threshold of a row from its candidates: every entry is above `lo`, and
// none of the row's other scores is.  Two lanes share a row (sums are
// combined with lane l ^ 32).  Newton steps from below on sqrt(F) - 1, F(t) =
// sum [(x - t)/2]_+^2 (the norm of a vector of convex non-negative functions
// of t, so convex and decreasing): a step from a point with F >= 1 stays at or
// below the root (bisection takes over if rounding lands above it).  Exact finish: when the closed-form root of {x > t} lies below
// the set's smallest member, that set is the support and the root is tau.
// Sums in fp64.  A step from a point above the root (rounding) is a Newton
// step too: the tangent of a convex decreasing function meets zero at or
// below the root.  Returns tau; lanes with active == false only take part in
// the exchanges.
template <class Src>
__device__ __forceinline__ double solve_candidates(const Src& src, double mx, double lo, double hi,
                                                   bool active) {
    double t = lo, result = lo;
    bool done = !active;
    for (int it = 0; it < kMaxIter; ++it) {
        if (__ballot(!done) == 0) break;
        // over {x > t}, with y = x - mx: count, sum y, sum y^2, smallest x
        int c = 0;
        double S1 = 0, S2 = 0;
        float mn = __builtin_inff();
        if (!done) {
            src.each([&](float x) {
                const bool on = (double)x > t;
                const double y = on ? (double)x - mx : 0.0;
                c += on ? 1 : 0;
                S1 += y;
                S2 = fma(y, y, S2);
                mn = fminf(mn, on ? x : __builtin_inff());
            });
        }
        c = pair_sum(c);
        S1 = pair_sum(S1);
        S2 = pair_sum(S2);
        mn = pair_min(mn);
        if (done) continue;
        const double C = (double)c, u = t - mx;
        // f(t) = sum ((y - u)/2)^2 - 1 and -f'(t) = sum (y - u)/2 over the set
        const double f = 0.25 * (S2 - 2.0 * u * S1 + C * u * u) - 1.0;
        const double F1 = 0.5 * (S1 - C * u);
        if (f >= 0.0 && c > 0) {
            lo = t;
            const double disc = fmax(S1 * S1 - C * (S2 - 4.0), 0.0);
            const double ts = mx + (S1 - sqrt(disc)) / C;
            if (ts < (double)mn) {
                result = fmax(ts, t);
                done = true;
                continue;
            }
            // Newton step on sqrt(F) - 1 (F = f + 1 = |g|^2, g = [(x - t)/2]_+):
            // the norm of g is convex and decreasing in t too, closer to
            // linear than F, so the step from below is longer (by up to 2x
            // while F >> 1) and still stays at or below the root
            const double rF = sqrt(f + 1.0);
            double tn = t + 2.0 * rF * (rF - 1.0) / F1;
            if (!(tn > lo && tn < hi)) tn = 0.5 * (lo + hi);
            t = tn;
        } else {
            hi = t;
            double tn = (F1 > 0.0) ? t + f / F1 : 0.5 * (lo + hi);
            if (!(tn > lo && tn < hi)) tn = 0.5 * (lo + hi);
            t = tn;
        }
        if (hi - lo <= 1e-12 * fmax(1.0, fabs(t))) {
            result = 0.5 * (lo + hi);
            done = true;
        }
    }
    if (!done) result = 0.5 * (lo + hi);
    return result;
}

// General alpha: tau of a candidate list (two lanes per row, sums combined
// with lane l ^ 32) by Newton steps from below on F = sum p, F1 = sum p/u
// with a bisection guard (newton_or_bisect).  *lo_out (optional) receives
// the last point with f >= 0, a lower bound on the list's threshold.
template <class Src>
__device__ __forceinline__ float solve_candidates_gen(const Src& src, float lo, float hi, bool active,
                                                      const AlphaMap& am, float* lo_out = nullptr) {
    float t = lo, result = lo;
    bool done = !active;
    for (int it = 0; it < kMaxIter; ++it) {
        if (__ballot(!done) == 0) break;
        float F = 0.f, F1 = 0.f;
        if (!done) {
            src.each([&](float x) {
                const float u = am.am1 * (x - t);
                if (u > 0.f) {
                    const float q = am.pw1(u);  // p / u
                    F = fmaf(q, u, F);
                    F1 += q;
                }
            });
        }
        F += __shfl_xor(F, 32, kWave);
        F1 += __shfl_xor(F1, 32, kWave);
        if (done) continue;
        bool fin;
        const float tn = newton_or_bisect(t, F, F1, lo, hi, &fin, am);
        if (fin) {
            result = tn;
            done = true;
        } else if (hi - lo <= 4e-7f * fmaxf(1.0f, fabsf(t))) {
            result = 0.5f * (lo + hi);
            done = true;
        } else {
            t = tn;
        }
    }
    if (!done) result = 0.5f * (lo + hi);
    if (lo_out) *lo_out = lo;
    return result;
}

// Workgroups per CU of the score-statistics sweep (three fit in the register
// file at <= 168 VGPRs).
constexpr int kStatsOcc = 3;
// Ring stages (pairs of tiles in flight + 1) of the score-statistics sweep.
template <typename T, int D>
struct StatsCfg {
    static constexpr int kS = (sizeof(T) == 2 && D == 64) ? 3 : (sizeof(T) == 2) ? 2 : ((D == 128) ? 2 : 3);
};
// Ring stages and workgroups per CU of the candidate sweeps (bf16, d = 128: a
// one-stage ring leaves room in LDS for two workgroups per CU, whose sweeps
// then hide each other's loads).
template <typename T, int D>
struct CollectCfg {
    static constexpr int kS = (D == 128) ? 1 : 2;
    static constexpr int kOcc = (sizeof(T) == 2) ? 2 : 1;
};

constexpr int kTop4 = 4;  // tile maxima kept per lane half per row

// Per-row and per-tile state of a 128-row block, kept in LDS across the
// phases of the forward (score statistics, threshold solve, output).
template <int TCMAX>
struct BlockLds {
    uint16_t list[TCMAX];         // the tile list of the current sweep
    float um_s[2][TCMAX];         // largest score per (64-row half, key tile)
    float row_m[kBR], row_lo[kBR], row_tau[kBR];
    uint32_t maskw[2][TCMAX / 32];
    int nlist_s, flag_s, vover_s;
};

// ------------------------------------------------------------ kernel 1a
// Dense sweep: per row the top tile maxima (-> tau_lo and the maximum) and
// per (64-row half, tile) the largest raw score.
// CAUSAL: the instance for the causal mask (its list-free sweep covers the
// tiles up to the diagonal); the other serves no mask and the window mask
// (which always takes the list).  Separate instances keep each loop's code
// as it is alone.
// keep: also leave each row's maximum and bound, and the tile maxima (raw),
// in the block's LDS state for the solve that follows in the same workgroup.
template <typename T, int D, int TCMAX, bool CAUSAL>
__device__ __forceinline__ void stats_phase(const FwdParams& p, int bh, int r0,
                                            const typename Ops<T, D>::template QOp<2>& qop, T* ring,
                                            BlockLds<TCMAX>& bl, bool keep) {
    constexpr int S = StatsCfg<T, D>::kS;
    uint16_t* const list = bl.list;
    float(&umax)[2][TCMAX] = bl.um_s;
    int& nlist_s = bl.nlist_s;
    // the per-row lists are merged through the ring once the sweep is over
    typedef float StRow[kBR][2 * kTop4];
    static_assert(sizeof(float) * 2 * kBR * 2 * kTop4 <= sizeof(T) * S * 2 * 64 * D, "merge space");
    StRow* st = reinterpret_cast<StRow*>(ring);

    const int t = threadIdx.x, w = wave_id(), qh = w & 1, kh = w >> 1;
    const int l = lane_id(), m = l & 31, h = l >> 5;
    const int R0 = r0 + 64 * qh;
    const Geom g = {p.L, p.mode, p.W};
    const T* Kh = reinterpret_cast<const T*>(p.k) + (size_t)bh * p.L * D;

    for (int i = t; i < 2 * TCMAX; i += kNT) (&umax[0][0])[i] = neg_inf();
    // the workgroup's tiles are the first dense_nt (no mask: all; causal: up
    // to the diagonal), all inside L: the list-free sweep
    const bool dense = p.L % kBC == 0 && r0 + kBR <= p.L &&
                       (CAUSAL ? p.mode == 1 : (p.mode == 0 && p.Tc % 2 == 0));
    if (w == 0 && !dense) {
        const int n = build_list(list, p.Tc, [&](int J) {
            return (tile_class(J, r0, g) != kSkip ? 1 : 0) | (tile_class(J, r0 + 64, g) != kSkip ? 2 : 0);
        });
        if (l == 0) nlist_s = n;
    }
    __syncthreads();

    float top[2][kTop4];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int i = 0; i < kTop4; ++i) top[qb][i] = neg_inf();

    auto tile_stats = [&](int J, int, f32x16(&acc)[2][2]) {
        float wm = neg_inf();
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            float tm = neg_inf();
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) tm = fmaxf(tm, acc[kb][qb][r]);
            float x = tm;
#pragma unroll
            for (int i = 0; i < kTop4; ++i) {
                const float hi = fmaxf(top[qb][i], x);
                x = fminf(top[qb][i], x);
                top[qb][i] = hi;
            }
            wm = fmaxf(wm, tm);
        }
        wm = wave_max_dpp(wm);
        if (l == 0) umax[qh][J] = wm;
    };
    if (dense) dense_sweep<T, D, S, CAUSAL>(CAUSAL ? r0 / kBC + 2 : p.Tc, Kh, ring, qop, R0, g, tile_stats);
    else ring_sweep<T, D, S>(list, nlist_s, Kh, ring, qop, R0, g, tile_stats);

    // merge the four lists of each row (two lane halves x two key parities)
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        float other[kTop4];
#pragma unroll
        for (int i = 0; i < kTop4; ++i) other[i] = __shfl_xor(top[qb][i], 32, kWave);
        if (h == 0) {
            float* e = &st[kh][qh * 64 + qb * 32 + m][0];
#pragma unroll
            for (int i = 0; i < kTop4; ++i) {
                e[i] = top[qb][i];
                e[kTop4 + i] = other[i];
            }
        }
    }
    __syncthreads();
    const int srow = qh * 64 + kh * 32 + m;
    const int grow = r0 + srow;
    if (h == 0 && grow < p.L) {
        float v[4 * kTop4];
#pragma unroll
        for (int i = 0; i < 2 * kTop4; ++i) {
            v[i] = st[0][srow][i] * p.scale;
            v[2 * kTop4 + i] = st[1][srow][i] * p.scale;
        }
        sort_desc(v);
        const float lo = p.gen ? tau_lower_gen(v, p.am) : tau_of_sorted(v);
        reinterpret_cast<float2*>(p.rowstat)[(size_t)bh * p.L + grow] = make_float2(v[0], lo);
        if (keep) {
            bl.row_m[srow] = v[0];
            bl.row_lo[srow] = lo;
        }
    } else if (h == 0 && keep) {
        bl.row_m[srow] = neg_inf();
        bl.row_lo[srow] = __builtin_inff();
    }
    for (int i = t; i < 2 * p.Tc; i += kNT) {
        const int hh = i / p.Tc, J = i % p.Tc;
        const int I = r0 / 64 + hh;
        if (I < p.Tr64) p.umax[((size_t)bh * p.Tr64 + I) * p.Tc + J] = umax[hh][J];
    }
}

template <typename T, int D, int TCMAX, bool CAUSAL>
__global__ __launch_bounds__(kNT, kStatsOcc) void fwd_stats_kernel(FwdParams p) {
    using O = Ops<T, D>;
    __shared__ __attribute__((aligned(16))) T ring[StatsCfg<T, D>::kS * 2 * 64 * D];
    __shared__ BlockLds<TCMAX> bl;
    int bh, r0;
    decode_item(blockIdx.x, p.BH, p.nQ, p.mode != 0, bh, r0);
    typename O::template QOp<2> qop;
    O::load_q(qop, reinterpret_cast<const T*>(p.q) + (size_t)bh * p.L * D, r0 + 64 * (wave_id() & 1), p.L);
    stats_phase<T, D, TCMAX, CAUSAL>(p, bh, r0, qop, ring, bl, false);
}

// O of a block's rows from their candidate lists: O_i = sum over the entries
// above tau_i of p(s) V_key (exactly the output over the non-null blocks,
// since every score of a row outside its list is at or below tau), fp32
// products and sums in list order.  D / 32 lanes per row, each with 32
// elements of d; the lanes of a row load each entry's V row piece by
// 16-byte loads, kB entries in flight.
// GV: in the same pass, G.V (the derivatives g = dA/dS as weights) into
// p.gv and their row sums into p.gsum; each V row is read once for both.
template <typename T, int D, bool GV>
__device__ __forceinline__ void gather_rows(const FwdParams& p, int bh, int r0, const u32x2* clist,
                                            const uint16_t (&cntq)[4][kBR], const float* row_tau) {
    constexpr int kLpr = D / 32;              // lanes per row
    constexpr int kRpp = kNT / kLpr;          // rows per pass
    constexpr int kVec = 16 / (int)sizeof(T); // elements per 16-byte load
    constexpr int kLd = 32 / kVec;            // loads per entry per lane
    constexpr int kB = sizeof(T) == 2 ? 4 : 2;
    const T* Vh = reinterpret_cast<const T*>(p.v) + (size_t)bh * p.L * D;
    const int t = threadIdx.x, part = t % kLpr;
    for (int rp = 0; rp < kBR; rp += kRpp) {
        const int row = rp + t / kLpr;
        if (r0 + row >= p.L) continue;
        const float tau = row_tau[row];
        const int n0 = cntq[0][row], n1 = n0 + cntq[1][row], n2 = n1 + cntq[2][row], n = n2 + cntq[3][row];
        float acc[32], accg[GV ? 32 : 1], gs = 0.0f;
#pragma unroll
        for (int j = 0; j < 32; ++j) acc[j] = 0.0f;
        if constexpr (GV) {
#pragma unroll
            for (int j = 0; j < 32; ++j) accg[j] = 0.0f;
        }
        // entry i of the row in list order (i < n)
        auto entry = [&](int i) -> u32x2 {
            const int qq = (i >= n0) + (i >= n1) + (i >= n2);
            const int c = i - (qq == 0 ? 0 : qq == 1 ? n0 : qq == 2 ? n1 : n2);
            return clist[(size_t)(4 * c + qq) * kBR + row];
        };
        // the entries of the next step are loaded while this step's V rows
        // are in flight, so a step waits for one round trip, not two
        u32x2 en[kB];
        if (n > 0) {
#pragma unroll
            for (int u = 0; u < kB; ++u) en[u] = entry(min(u, n - 1));
        }
        for (int i0 = 0; i0 < n; i0 += kB) {
            float a[kB], gw[kB];
            uint32_t key[kB];
            u32x2 ec[kB];
#pragma unroll
            for (int u = 0; u < kB; ++u) ec[u] = en[u];
#pragma unroll
            for (int u = 0; u < kB; ++u) {
                const u32x2 e = ec[u];
                const float sv = __builtin_bit_cast(float, e[0]);
                const bool live = i0 + u < n;
                if (p.gen) {
                    a[u] = live ? p.am.p(sv, tau) : 0.0f;
                    if constexpr (GV) gw[u] = live ? p.am.g(sv, tau) : 0.0f;
                } else {
                    const float dd = live ? 0.5f * fmaxf(sv - tau, 0.0f) : 0.0f;
                    a[u] = dd * dd;
                    if constexpr (GV) gw[u] = dd;
                }
                if constexpr (GV) gs += gw[u];
                key[u] = e[1];
            }
            u32x4 v[kB][kLd];
#pragma unroll
            for (int u = 0; u < kB; ++u)
#pragma unroll
                for (int j = 0; j < kLd; ++j)
                    v[u][j] = *reinterpret_cast<const u32x4*>(Vh + (size_t)key[u] * D + part * 32 + j * kVec);
            if (i0 + kB < n) {
#pragma unroll
                for (int u = 0; u < kB; ++u) en[u] = entry(min(i0 + kB + u, n - 1));
            }
#pragma unroll
            for (int u = 0; u < kB; ++u)
#pragma unroll
                for (int j = 0; j < kLd; ++j)
#pragma unroll
                    for (int e = 0; e < kVec; ++e) {
                        // (the element is copied out first: a bit_cast of an
                        // indexed vector element read element 0 here)
                        const uint32_t bits = v[u][j][sizeof(T) == 2 ? e >> 1 : e];
                        const float x = sizeof(T) == 2 ? __builtin_bit_cast(float, (bits >> ((e & 1) * 16)) << 16)
                                                       : __builtin_bit_cast(float, bits);
                        acc[j * kVec + e] = fmaf(a[u], x, acc[j * kVec + e]);
                        if constexpr (GV) accg[j * kVec + e] = fmaf(gw[u], x, accg[j * kVec + e]);
                    }
        }
        const size_t off = ((size_t)bh * p.L + r0 + row) * D + part * 32;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            f32x4 o4;
#pragma unroll
            for (int e = 0; e < 4; ++e) o4[e] = acc[4 * j + e];
            *reinterpret_cast<f32x4*>(p.o + off + 4 * j) = o4;
        }
        if constexpr (GV) {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                f32x4 g4;
#pragma unroll
                for (int e = 0; e < 4; ++e) g4[e] = accg[4 * j + e];
                *reinterpret_cast<f32x4*>(p.gv + off + 4 * j) = g4;
            }
            if (part == 0) p.gsum[(size_t)bh * p.L + r0 + row] = gs;
        }
    }
}

// ------------------------------------------------------------ kernel 1b
// Threshold of the 128 rows of a block from their score statistics.
//
// collect   sweep the tiles whose largest score beats the smallest bound of
//           the row half; every score above its row's bound goes to the
//           row's sub-list of the sweeping lane (a register takes the store
//           path only when some lane of the wave holds such a score in it).
//           Nothing at or below a lower bound on tau carries weight, so a row
//           whose four sub-lists all fit holds its whole support in them.
// solve     exact tau of every complete row (two lanes per row, fp64 sums in
//           list order); the tiles of its support are set in the block mask.
// overflow  rows whose sub-lists overflow (wide supports) take the histogram
//           initialisation of "AdaSplash-2: Faster Differentiable Sparse
//           Attention" (sec. 3.1, sec. 3.3 phase 2): one sweep bins every
//           score above the row's bound into 32 left-edge bins spanning
//           [bound, max]; the exact threshold tau_h of the binned scores
//           satisfies tau - w < tau_h <= tau (Proposition 3.1, w the bin
//           width).  A row whose scores above tau_h fit the lists is collected
//           again above tau_h and solved exactly; any other row is refined by
//           Halley-bisection sweeps on [tau_h, tau_h + w] (phase 3), and a
//           last sweep sets its tiles in the mask.
template <int D>
constexpr int kSolveRegs = D == 128 ? 8 : 16;  // candidates per lane held in registers
// and the next ones per lane in LDS: the score ring every caller of the solve
// passes holds at least 2 x 64 x D elements of T per stage, S stages, read as
// words over kNT threads (the keys of the register entries take kSolveRegs)
template <typename T, int D, int S>
constexpr int kSolveLds = (S * 2 * 64 * D * (int)sizeof(T) / (4 * kNT) - kSolveRegs<D>) < 16
                              ? S * 2 * 64 * D * (int)sizeof(T) / (4 * kNT) - kSolveRegs<D>
                              : 16;
constexpr int kHistBins = 32;

// The solve kernel writes O itself from the candidate lists when
// kGatherRatio * (list entries) < kGatherTileCost * (non-null tiles of its two
// 64-row blocks): a tile of the output pass (score recompute and product over
// 64 x 64 pairs) measured about 40 times the cost of one list entry's V row.
constexpr int kGatherRatio = 1;
constexpr int kGatherTileCost = 32;

// Row states of the solve kernel.
enum { kRowNone = 0, kRowCollect = 1, kRowSweep = 2, kRowDone = 3, kRowOver = 4 };

// LDS of the solve phase alone: per-row state, and the scratch of the
// overflow path (the histogram, then the sweep sums).  PACK: two 16-bit bin
// counts per word (bin 2i in the low half of word i, bin 2i + 1 in the high
// half), for rows of at most 65535 scores (the fused kernel: L <= 16384).
template <bool PACK>
struct SolveScratch {
    static constexpr int kPer = PACK ? 2 : 1;  // bins per word
    float row_hi[kBR];
    int rstate[kBR];
    uint16_t cntq[4][kBR];  // entries met per candidate sub-list
    int state_s;            // bit s set: some row of the block is in state s after the last solve
    int gwork_s;            // list entries of the block (the gather decision)
    union {
        uint32_t hist[kHistBins / kPer * kBR];  // counts [bin / kPer][row]
        struct {
            float t[kBR];
            int active[kBR];
            float part[kBR][2][4];
        } fb;
    };
    static constexpr int kHistWords = kHistBins / kPer * kBR;
    __device__ __forceinline__ void hist_add(int k, int row) {
        atomicAdd(&hist[(k / kPer) * kBR + row], PACK ? 1u << (16 * (k & 1)) : 1u);
    }
    __device__ __forceinline__ int hist_get(int k, int row) const {
        const uint32_t w = hist[(k / kPer) * kBR + row];
        return PACK ? (int)((w >> (16 * (k & 1))) & 0xffffu) : (int)w;
    }
};

// from_stats: the block's row statistics and raw tile maxima are already in
// bl (the score sweep ran in this workgroup); otherwise they are read from
// the workspace.  Returns whether it wrote O from the candidate lists.
template <typename T, int D, int TCMAX, int S, bool PACK>
__device__ __forceinline__ bool solve_phase(const FwdParams& p, int bh, int r0,
                                            const typename Ops<T, D>::template QOp<2>& qop, T* ring,
                                            SolveScratch<PACK>& ss, BlockLds<TCMAX>& bl, bool from_stats) {
    constexpr int WD = TCMAX / 32;
    uint16_t* const list = bl.list;
    float(&um_s)[2][TCMAX] = bl.um_s;
    uint16_t(&cntq)[4][kBR] = ss.cntq;
    int* const rstate = ss.rstate;
    float* const row_m = bl.row_m;
    float* const row_lo = bl.row_lo;
    float* const row_hi = ss.row_hi;
    float* const row_tau = bl.row_tau;
    uint32_t(&maskw)[2][WD] = bl.maskw;
    int& nlist_s = bl.nlist_s;
    int& flag_s = bl.flag_s;

    const int t = threadIdx.x, w = wave_id(), qh = w & 1, kh = w >> 1;
    const int l = lane_id(), m = l & 31, h = l >> 5;
    const int q = 2 * kh + h;  // this lane's sub-list of the rows it sweeps
    const size_t blk = (size_t)bh * p.nQ + r0 / kBR;
    const int R0 = r0 + 64 * qh;
    const Geom g = {p.L, p.mode, p.W};
    const T* Kh = reinterpret_cast<const T*>(p.k) + (size_t)bh * p.L * D;
    const int cap = p.cap < kCandCap ? p.cap : kCandCap;
    const int capq = cap >= 4 ? cap / 4 : 1;  // entries per sub-list
    u32x2* clist = p.clist + blk * kCandCap * kBR;
    const float2* rowstat = reinterpret_cast<const float2*>(p.rowstat) + (size_t)bh * p.L;

    // row statistics and the tile maxima of both row blocks
    if (t < kBR) {
        const bool valid = (r0 + t) < p.L;
        if (!from_stats) {
            const float2 rs = valid ? rowstat[r0 + t] : make_float2(neg_inf(), __builtin_inff());
            row_m[t] = rs.x;
            row_lo[t] = rs.y;
        }
        rstate[t] = valid ? kRowCollect : kRowNone;
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) cntq[qq][t] = 0;
    }
    for (int i = t; i < 2 * p.Tc; i += kNT) {
        const int hh = i / p.Tc, J = i - hh * p.Tc;
        const int I = r0 / 64 + hh;
        if (from_stats) um_s[hh][J] *= p.scale;
        else um_s[hh][J] = (I < p.Tr64) ? p.umax[((size_t)bh * p.Tr64 + I) * p.Tc + J] * p.scale : neg_inf();
    }
    for (int i = t; i < 2 * WD; i += kNT) (&maskw[0][0])[i] = 0u;
    __syncthreads();

    // tiles whose best score beats the smallest bound of the row half
    if (w == 0) {
        const float th0 = wave_min(row_lo[l]), th1 = wave_min(row_lo[64 + l]);
        const int n = build_list(list, p.Tc, [&](int J) {
            return (um_s[0][J] > th0 ? 1 : 0) | (um_s[1][J] > th1 ? 2 : 0);
        });
        if (l == 0) nlist_s = n;
    }
    __syncthreads();

    const int srow = qh * 64 + kh * 32 + m;  // the row this lane solves (with lane l ^ 32)

    // ---- collect the scores above each collecting row's bound
    // bin: scores past a sub-list's capacity go to the row's histogram over
    // [bound, max] (the overflow path adds the listed ones after the solve)
    auto collect = [&](bool bin) {
        float lr[2], hlo[2], hinv[2];
        int cc[2] = {0, 0};
        bool coll[2];
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            const int row = qh * 64 + qb * 32 + m;
            coll[qb] = rstate[row] == kRowCollect;
            lr[qb] = coll[qb] ? raw_threshold(row_lo[row], p.scale) : __builtin_inff();
            hlo[qb] = row_lo[row];
            hinv[qb] = coll[qb] ? (float)kHistBins / (row_m[row] - row_lo[row]) : 0.0f;
        }
        ring_sweep<T, D, S>(list, nlist_s, Kh, ring, qop, R0, g, [&](int J, int, f32x16(&acc)[2][2]) {
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
                const int row = qh * 64 + qb * 32 + m;
                // skip the 32 x 64 block when no lane holds a candidate in it
                float mx = neg_inf();
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, acc[kb][qb][r]);
                if (__builtin_amdgcn_ballot_w64(mx > lr[qb]) == 0) continue;
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const float x = acc[kb][qb][r];
                        if (x > lr[qb]) {
                            // past the capacity only the count goes on: it shows
                            // the overflow, and the list is not used
                            const int c = cc[qb];
                            if (c < capq) {
                                u32x2 e;
                                e[0] = __builtin_bit_cast(uint32_t, x * p.scale);
                                e[1] = (uint32_t)(J * kBC + kb * 32 + key_of_reg(r, h));
                                clist[(size_t)(4 * c + q) * kBR + row] = e;
                            } else if (bin) {
                                // (x * scale > bound, so the bin index is >= 0)
                                const int k = min((int)((x * p.scale - hlo[qb]) * hinv[qb]), kHistBins - 1);
                                ss.hist_add(k, row);
                            }
                            cc[qb] = c + 1;
                        }
                    }
            }
        });
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
            if (coll[qb]) cntq[q][qh * 64 + qb * 32 + m] = cc[qb];
        __syncthreads();
    };

    // ---- exact tau of the collecting rows whose sub-lists all fit
    auto solve = [&]() {
        if (t == 0) {
            ss.state_s = 0;
            ss.gwork_s = 0;
        }
        const bool open = rstate[srow] == kRowCollect;
        const int a0 = cntq[h][srow], a1 = cntq[2 + h][srow];
        const int b0 = cntq[h ^ 1][srow], b1 = cntq[2 + (h ^ 1)][srow];
        const bool act = open && max(max(a0, a1), max(b0, b1)) <= capq;
        const int n = act ? a0 + a1 + b0 + b1 : 1;
        // (the score ring is idle between sweeps)
        RegSrc<kSolveRegs<D>, kSolveLds<T, D, S>> src;
        src.load(CandSrc{clist + srow, act ? a0 : 0, act ? a1 : 0, h}, reinterpret_cast<uint32_t*>(ring) + t);
        const double mx = row_m[srow];
        const float tr = p.gen ? solve_candidates_gen(src, row_lo[srow], p.am.hi(row_m[srow], (float)n), act, p.am)
                               : (float)solve_candidates(src, mx, row_lo[srow], mx - 2.0 / sqrt((double)n), act);
        if (act) {
            // the tiles of the support (a lane meets its entries in tile order)
            int lastJ = -1;
            const int na = a0 + a1;
            auto mark = [&](float x, uint32_t key) {
                if (x > tr) {
                    const int J = (int)(key >> 6);
                    if (J != lastJ) atomicOr(&maskw[qh][J >> 5], 1u << (J & 31));
                    lastJ = J;
                }
            };
#pragma unroll
            for (int k = 0; k < kSolveRegs<D>; ++k) mark(src.v[k], src.key(k));
            // the rest from the workspace, four entries loaded at once from
            // clamped slots (inside the lists)
            for (int i = kSolveRegs<D>; __builtin_amdgcn_ballot_w64(i < na) != 0; i += 4) {
                u32x2 e[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) e[u] = src.src.entry(max(min(i + u, na - 1), 0));
#pragma unroll
                for (int u = 0; u < 4; ++u)
                    if (i + u < na) mark(__builtin_bit_cast(float, e[u][0]), e[u][1]);
            }
            if (h == 0) {
                row_tau[srow] = tr;
                rstate[srow] = kRowDone;
            }
        } else if (open && h == 0) {
            rstate[srow] = kRowOver;
        }
        if (h == 0) {
            atomicOr(&ss.state_s, 1 << rstate[srow]);
            const int ne = a0 + a1 + b0 + b1;
            if (ne != 0) atomicAdd(&ss.gwork_s, kGatherRatio * ne);
        }
        __syncthreads();
    };

    // any row of the block in state st?
    auto any_row = [&](int st) -> bool {
        if (t == 0) flag_s = 0;
        __syncthreads();
        if (t < kBR && rstate[t] == st) atomicOr(&flag_s, 1);
        __syncthreads();
        return flag_s != 0;
    };

    // the histogram of the overflow path is built during the first collect
    // (the ring sweep's first barrier orders the clearing before its atomics)
    for (int i = t; i < ss.kHistWords; i += kNT) ss.hist[i] = 0u;
    collect(true);
    solve();

    // (no row overflowed: no row can be in the sweep state below)
    const bool overflowed = (ss.state_s >> kRowOver) & 1;
    if (overflowed) {
        // ---- histogram of the scores above the bound of each overflowing
        // row: the collect binned the scores past the lists' capacity; add
        // the listed ones (entry i of sub-list qq of a row sits at
        // (4 i + qq) kBR + row, so the threads walk the lists in order)
        // (kNT is a multiple of kBR, so a thread keeps its row; every slot
        // read lies inside the lists, so four loads go out at once)
        static_assert(kNT % kBR == 0, "one row per thread");
        {
            const int row = t % kBR;
            const bool over = rstate[row] == kRowOver;
            const float rlo = row_lo[row], rinv = (float)kHistBins / (row_m[row] - row_lo[row]);
            const int nE = 4 * capq * kBR;
            for (int e0 = t; e0 < nE; e0 += 4 * kNT) {
                float sv[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) sv[u] = __builtin_bit_cast(float, clist[min(e0 + u * kNT, nE - 1)][0]);
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int e = e0 + u * kNT, qq = (e / kBR) & 3, i = e / (4 * kBR);
                    if (e < nE && over && i < (int)cntq[qq][row]) {
                        const int k = min((int)((sv[u] - rlo) * rinv), kHistBins - 1);
                        ss.hist_add(k, row);
                    }
                }
            }
        }
        __syncthreads();
        // tau_h from the bin counts (one thread per row), the bracket
        // [tau_h, tau_h + w], and whether the scores above tau_h fit the lists
        if (t < kBR && rstate[t] == kRowOver) {
            const double lo = row_lo[t], mx = row_m[t];
            const double wd = (mx - lo) / kHistBins;
            double th;
            if (!p.gen) {
                // the sorting solve on the bins, from the top (each bin's
                // scores stand at its left edge)
                double S0 = 0.0, S1 = 0.0, S2 = 0.0, best = -2.0;
                for (int k = kHistBins - 1; k >= 0; --k) {
                    const double H = (double)ss.hist_get(k, t);
                    if (H == 0.0) continue;
                    const double y = lo + k * wd - mx;
                    S0 += H;
                    S1 += H * y;
                    S2 += H * y * y;
                    const double disc = S1 * S1 - S0 * (S2 - 4.0);
                    if (disc < 0.0) continue;
                    const double tk = (S1 - sqrt(disc)) / S0;
                    if (tk <= y) best = tk;
                }
                th = mx + best;
            } else {
                // bisection on the binned normaliser
                double a = lo - wd, b = mx;
                for (int it = 0; it < 60; ++it) {
                    const double mid = 0.5 * (a + b);
                    double F = 0.0;
                    for (int k = 0; k < kHistBins; ++k) {
                        const int H = ss.hist_get(k, t);
                        const double u = (double)p.am.am1 * (lo + k * wd - mid);
                        if (H > 0 && u > 0.0) F += H * (p.am.lin ? u : pow(u, (double)p.am.e));
                    }
                    if (F >= 1.0) a = mid; else b = mid;
                }
                th = a;
            }
            // margins for the fp32 binning arithmetic
            const double mg = 1e-6 * fmax(1.0, fabs(th));
            const float tlo = (float)fmax(th - mg, lo);
            const float thi = (float)fmin(th + wd + mg, mx);
            int above = 0;
            const int k0 = max((int)floor((tlo - lo) / wd) - 1, 0);
            for (int k = k0; k < kHistBins; ++k) above += ss.hist_get(k, t);
            row_lo[t] = fmaxf(row_lo[t], tlo);
            row_hi[t] = thi;
            rstate[t] = (above <= 3 * capq) ? kRowCollect : kRowSweep;
        }
        __syncthreads();
        if (any_row(kRowCollect)) {
            collect(false);
            solve();
            // rows still overflowing keep the histogram bracket
            if (t < kBR && rstate[t] == kRowOver) rstate[t] = kRowSweep;
            __syncthreads();
        }
    }

    // ---- refinement sweeps for rows whose lists overflowed: Newton steps
    // from below on F^(alpha-1) - 1 (newton_or_bisect), from the two sums F =
    // sum p and F1 = sum p/u; at alpha = 1.5 that is sqrt(F) - 1, the 2-norm
    // of the g_i less 1, which is exactly linear in tau while the support
    // stays fixed, so the steps land on tau once the support is found.
    const bool swept = overflowed && any_row(kRowSweep);
    if (swept) {
        float* const fb_t = ss.fb.t;
        int* const fb_active = ss.fb.active;
        float(&fb_part)[kBR][2][4] = ss.fb.part;
        if (h == 0) {
            fb_active[srow] = rstate[srow] == kRowSweep ? 1 : 0;
            fb_t[srow] = row_lo[srow];
        }
        __syncthreads();
        for (int it = 0; it < kFbMaxIter; ++it) {
            float tq[2], lr[2];
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
                const int row = qh * 64 + qb * 32 + m;
                tq[qb] = fb_t[row];
                lr[qb] = fb_active[row] != 0 ? raw_threshold(tq[qb], p.scale) : __builtin_inff();
            }
            float sf[2] = {0.f, 0.f}, sf1[2] = {0.f, 0.f};
            const float hs = 0.5f * p.scale;
            const float hc[2] = {-0.5f * tq[0], -0.5f * tq[1]};
            ring_sweep<T, D, S>(list, nlist_s, Kh, ring, qop, R0, g, [&](int, int, f32x16(&acc)[2][2]) {
#pragma unroll
                for (int qb = 0; qb < 2; ++qb) {
                    float mx = neg_inf();
#pragma unroll
                    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, acc[kb][qb][r]);
                    if (__builtin_amdgcn_ballot_w64(mx > lr[qb]) == 0) continue;
                    if (p.gen) {
#pragma unroll
                        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                            for (int r = 0; r < 16; ++r) {
                                const float x = acc[kb][qb][r];
                                if (x > lr[qb]) {
                                    // F = sum p, F1 = sum p/u
                                    const float u = p.am.am1 * (x * p.scale - tq[qb]);
                                    const float pu = p.am.pw1(u);  // p / u
                                    sf[qb] = fmaf(pu, u, sf[qb]);
                                    sf1[qb] += pu;
                                }
                            }
                    } else {
                        // g = [(s - t)/2]_+, F = sum g^2, F1 = sum g: three
                        // operations per score, no branch
#pragma unroll
                        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                            for (int r = 0; r < 16; ++r) {
                                const float gg = fmaxf(fmaf(acc[kb][qb][r], hs, hc[qb]), 0.0f);
                                sf[qb] = fmaf(gg, gg, sf[qb]);
                                sf1[qb] += gg;
                            }
                    }
                }
            });
            // combine the two lane halves, then the two key parities
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
                sf[qb] += __shfl_xor(sf[qb], 32, kWave);
                sf1[qb] += __shfl_xor(sf1[qb], 32, kWave);
                if (h == 0) {
                    const int row = qh * 64 + qb * 32 + m;
                    fb_part[row][kh][0] = sf[qb];
                    fb_part[row][kh][1] = sf1[qb];
                }
            }
            if (t == 0) flag_s = 0;
            __syncthreads();
            if (h == 0 && fb_active[srow]) {
                const float F = fb_part[srow][0][0] + fb_part[srow][1][0];
                const float F1 = fb_part[srow][0][1] + fb_part[srow][1][1];
                float lo = row_lo[srow], hi = row_hi[srow], tc = fb_t[srow];
                // (at alpha = 1.5, F1 = sum g is sum p/u of the general map)
                bool fin;
                const float tn = newton_or_bisect(tc, F, F1, lo, hi, &fin, p.am);
                if (fin || hi - lo <= 4e-7f * fmaxf(1.0f, fabsf(tc))) {
                    fb_active[srow] = 0;
                    row_tau[srow] = fin ? tn : 0.5f * (lo + hi);
                } else {
                    fb_t[srow] = tn;
                    atomicOr(&flag_s, 1);
                }
                row_lo[srow] = lo;
                row_hi[srow] = hi;
            }
            __syncthreads();
            if (!flag_s) break;
        }
        // rows still active after the cap take their bracket midpoint
        if (h == 0 && fb_active[srow]) row_tau[srow] = 0.5f * (row_lo[srow] + row_hi[srow]);
        __syncthreads();
        // mark the tiles of the swept rows: a tile is set when some score of
        // such a row exceeds its tau (compared as raw products)
        float lr[2];
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            const int row = qh * 64 + qb * 32 + m;
            lr[qb] = rstate[row] == kRowSweep ? raw_threshold(row_tau[row], p.scale) : __builtin_inff();
        }
        ring_sweep<T, D, S>(list, nlist_s, Kh, ring, qop, R0, g, [&](int J, int, f32x16(&acc)[2][2]) {
            bool any = false;
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
                float mx = neg_inf();
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, acc[kb][qb][r]);
                any |= mx > lr[qb];
            }
            if (__ballot(any) != 0 && l == 0) atomicOr(&maskw[qh][J >> 5], 1u << (J & 31));
        });
    }
    __syncthreads();

    // ---- O straight from the candidate lists when every row has one and the
    // lists are short next to the tiles the output pass would sweep
    bool gathered = false;
    if (p.gather) {
        gathered = !swept;
        if (gathered) {
            // the solve summed the list entries; less the tiles' cost
            if (t < 2 * WD) {
                const int pc = __popc((&maskw[0][0])[t]);
                if (pc != 0) atomicAdd(&ss.gwork_s, -kGatherTileCost * pc);
            }
            __syncthreads();
            gathered = ss.gwork_s < 0;
        }
        if (gathered) {
            if (p.gv != nullptr) gather_rows<T, D, true>(p, bh, r0, clist, cntq, row_tau);
            else gather_rows<T, D, false>(p, bh, r0, clist, cntq, row_tau);
        }
        if (t == 0 && p.ostate != nullptr) p.ostate[blk] = gathered ? 1 : 0;
    }

    // ---- outputs: tau and the packed mask of both 64-row blocks
    if (t < kBR && r0 + t < p.L) p.tau[(size_t)bh * p.L + r0 + t] = row_tau[t];
    for (int i = t; i < 2 * p.Wd; i += kNT) {
        const int hh = i / p.Wd, wd = i % p.Wd;
        const int I = r0 / 64 + hh;
        if (I < p.Tr64) p.mask[((size_t)bh * p.Tr64 + I) * p.Wd + wd] = maskw[hh][wd];
    }
    return gathered;
}

template <typename T, int D, int TCMAX>
__global__ __launch_bounds__(kNT, (CollectCfg<T, D>::kOcc)) void fwd_solve_kernel(FwdParams p) {
    using O = Ops<T, D>;
    __shared__ __attribute__((aligned(16))) T ring[CollectCfg<T, D>::kS * 2 * 64 * D];
    __shared__ SolveScratch<false> ss;
    __shared__ BlockLds<TCMAX> bl;
    int bh, r0;
    decode_item(blockIdx.x, p.BH, p.nQ, p.mode != 0, bh, r0);
    typename O::template QOp<2> qop;
    O::load_q(qop, reinterpret_cast<const T*>(p.q) + (size_t)bh * p.L * D, r0 + 64 * (wave_id() & 1), p.L);
    solve_phase<T, D, TCMAX, CollectCfg<T, D>::kS>(p, bh, r0, qop, ring, ss, bl, false);
}

// ------------------------------------------------------------ kernel 2
template <typename T, int D, bool GEN>
__global__ __launch_bounds__(kNT, 1) void fwd_out_kernel(FwdParams p) {
    using O = Ops<T, D>;
    constexpr int NBUF = (sizeof(T) == 4 && D == 128) ? 1 : 2;
    constexpr int kKV = NBUF * 2 * (O::kKTile + O::kVTile);
    constexpr int kRed = 2 * 64 * (D + 4);  // floats for the O reduction
    constexpr int kBytes = (kKV * (int)sizeof(T) > kRed * 4) ? kKV * (int)sizeof(T) : kRed * 4;
    __shared__ __attribute__((aligned(16))) unsigned char smem[kBytes];
    __shared__ uint16_t list[kMaxTc];
    __shared__ uint32_t mw[2][kMaxTc / 32];
    __shared__ int nlist_s;

    T* kbuf = reinterpret_cast<T*>(smem);
    T* vbuf = kbuf + NBUF * 2 * O::kKTile;

    const int t = threadIdx.x, w = wave_id(), qh = w & 1, kh = w >> 1;
    const int l = lane_id(), m = l & 31, h = l >> 5;
    int bh, r0;
    decode_item(blockIdx.x, p.BH, p.nQ, p.mode != 0, bh, r0);
    if (p.ostate != nullptr && p.ostate[(size_t)bh * p.nQ + r0 / kBR]) return;  // O already written
    const int R0 = r0 + 64 * qh;
    const Geom g = {p.L, p.mode, p.W};
    const size_t head_off = (size_t)bh * p.L * D;
    const T* Qh = reinterpret_cast<const T*>(p.q) + head_off;
    const T* Kh = reinterpret_cast<const T*>(p.k) + head_off;
    const T* Vh = reinterpret_cast<const T*>(p.v) + head_off;

    for (int i = t; i < 2 * p.Wd; i += kNT) {
        const int hh = i / p.Wd, wd = i % p.Wd;
        const int I = r0 / 64 + hh;
        mw[hh][wd] = (I < p.Tr64) ? p.mask[((size_t)bh * p.Tr64 + I) * p.Wd + wd] : 0u;
    }
    __syncthreads();
    if (w == 0) {
        const int n = build_list(list, p.Tc, [&](int J) {
            return (int)((mw[0][J >> 5] >> (J & 31)) & 1u) | (int)(((mw[1][J >> 5] >> (J & 31)) & 1u) << 1);
        });
        if (l == 0) nlist_s = n;
    }
    typename O::template QOp<2> qop;
    O::load_q(qop, Qh, R0, p.L);
    float tq[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        const int row = R0 + qb * 32 + m;
        tq[qb] = (row < p.L) ? p.tau[(size_t)bh * p.L + row] : __builtin_inff();
    }
    typename O::template OAcc<2> oa;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
#pragma unroll
            for (int i = 0; i < 16; ++i) oa.o[db][qb][i] = 0.f;
    __syncthreads();

    sweep<T, D, NBUF, true>(list, nlist_s, Kh, Vh, kbuf, vbuf, qop, R0, g,
                            [&](int, int, f32x16(&acc)[2][2], const T* vt) {
        // 4A = [s - tau]_+^2 with s = scale * (Q.K) (general alpha: 4 p)
        if constexpr (GEN) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int qb = 0; qb < 2; ++qb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) acc[kb][qb][r] = 4.0f * p.am.p(acc[kb][qb][r] * p.scale, tq[qb]);
        } else {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int qb = 0; qb < 2; ++qb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const float dd = fmaxf(acc[kb][qb][r] * p.scale - tq[qb], 0.0f);
                        acc[kb][qb][r] = dd * dd;
                    }
        }
        const bool on[2] = {true, true};
        O::pv(oa, vt, acc, on);
    });

    // ---- reduce the two key parities and write O = (1/4) sum 4A V
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
                    const int q = qb * 32 + m, d = db * 32 + 8 * r4 + 4 * h;
                    *reinterpret_cast<f32x4*>(red + (qh * 64 + q) * kRS + d) = v4;
                }
    }
    __syncthreads();
    if (kh == 0) {
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
                    for (int e = 0; e < 4; ++e) v4[e] = 0.25f * (oa.o[db][qb][4 * r4 + e] + o2[e]);
                    *reinterpret_cast<f32x4*>(p.o + ((size_t)bh * p.L + row) * D + d) = v4;
                }
            }
    }
}

// ------------------------------------------------------------ kernel 2, bf16
// Output over the non-null tiles for bf16 inputs.  Each of the four waves
// owns 32 query rows and every key of a tile, so nothing is reduced across
// waves.  K (natural, swizzled) and V (transposed to V^T[d][key]) are staged
// per tile through registers into two LDS buffers.  O^T += V^T A^T runs on
// fp16 MFMA, the recipe of "AdaSplash-2: Faster Differentiable Sparse
// Attention" sec. 3.3 phase 4 (A and the V tile cast to fp16): A <= 1 keeps 11
// significant bits in fp16, and bf16 V converts exactly within fp16 range.  A
// workgroup that meets a V entry beyond that range redoes its rows with A
// split into bf16 hi + lo against bf16 V.
template <int D>
struct OutLds {
    __bf16 kbuf[2][Ops<__bf16, D>::kKTile];
    uint16_t vbuf[2][D * Ops<__bf16, D>::kVRow];  // fp16 or bf16 bits
};

// The block's rows from the tiles whose bits are set in mw0 / mw1 (its two
// 64-row blocks' mask words).  wk = 1: the derivatives g = dA/dS as weights
// (<= 1 like A), into p.gv, and their row sums into p.gsum.
template <int D, bool GEN>
__device__ __forceinline__ void out_phase_bf16(const FwdParams& p, int bh, int r0, OutLds<D>& ol,
                                               const uint32_t* mw0, const uint32_t* mw1, uint16_t* list,
                                               int& nlist_s, int& vover_s, const float* tau_lds, int wk = 0) {
    using O = Ops<__bf16, D>;
    constexpr int kVRow = O::kVRow;
    constexpr int kKPer = O::kChunks / kNT;  // K chunks per thread per tile
    static_assert(O::kChunks % kNT == 0 && O::kVUnits <= kNT, "staging split");
    auto& kbuf = ol.kbuf;
    auto& vbuf = ol.vbuf;

    const int t = threadIdx.x, w = wave_id();
    const int l = lane_id(), m = l & 31, h = l >> 5;
    const int R0 = r0 + 32 * w;  // this wave's rows
    const int hh = w >> 1;       // their 64-row block
    const Geom g = {p.L, p.mode, p.W};
    const size_t head_off = (size_t)bh * p.L * D;
    const __bf16* Qh = reinterpret_cast<const __bf16*>(p.q) + head_off;
    const __bf16* Kh = reinterpret_cast<const __bf16*>(p.k) + head_off;
    const __bf16* Vh = reinterpret_cast<const __bf16*>(p.v) + head_off;

    if (t == 0) vover_s = 0;
    __syncthreads();
    if (w == 0) {
        const int n = build_list(list, p.Tc, [&](int J) {
            return (int)((mw0[J >> 5] >> (J & 31)) & 1u) | (int)(((mw1[J >> 5] >> (J & 31)) & 1u) << 1);
        });
        if (l == 0) nlist_s = n;
    }
    typename O::template QOp<1> qop;
    O::load_q(qop, Qh, R0, p.L);
    const float tq = (R0 + m >= p.L) ? __builtin_inff()
                     : tau_lds != nullptr ? tau_lds[R0 + m - r0] : p.tau[(size_t)bh * p.L + R0 + m];
    __syncthreads();
    const int n = nlist_s;

    u32x4 kr[kKPer];
    typename O::VRegs vr;
    auto load = [&](int e) {
        const int c0 = (list[e] & 0xfff) * kBC;
#pragma unroll
        for (int i = 0; i < kKPer; ++i) kr[i] = O::load_k_chunk(Kh, c0, g.L, t + kNT * i);
        if (t < O::kVUnits) vr = O::load_v_unit(Vh, c0, g.L, t);
    };
    // V^T row d holds keys 4kg .. 4kg + 3 of unit (kg, dg) at 4kg; fp16 when
    // F16 (returns whether an entry left fp16 range), bf16 otherwise
    auto store = [&](int buf, bool f16) -> bool {
#pragma unroll
        for (int i = 0; i < kKPer; ++i) O::store_k_chunk(kbuf[buf], t + kNT * i, kr[i]);
        bool over = false;
        if (t < O::kVUnits) {
            if (!f16) {
                O::store_v_unit(reinterpret_cast<__bf16*>(vbuf[buf]), t, vr);
            } else {
                const int kg = t % (kBC / 4), dg = t / (kBC / 4);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    uint32_t hw[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const uint32_t bits = (vr.r[i][e >> 1] >> ((e & 1) * 16)) & 0xffffu;
                        const float f = __builtin_bit_cast(float, bits << 16);
                        over |= fabsf(f) > 65504.0f;
                        hw[i] = __builtin_bit_cast(uint16_t, (_Float16)f);
                    }
                    u32x2 pk;
                    pk[0] = hw[0] | (hw[1] << 16);
                    pk[1] = hw[2] | (hw[3] << 16);
                    *reinterpret_cast<u32x2*>(&vbuf[buf][(dg * 8 + e) * kVRow + 4 * kg]) = pk;
                }
            }
        }
        return over;
    };

    typename O::template OAcc<1> oa;
    float gs = 0.0f;
    auto run = [&](bool f16) {
        gs = 0.0f;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int i = 0; i < 16; ++i) oa.o[db][0][i] = 0.f;
        if (n == 0) return;
        bool over = false;
        load(0);
        over |= store(0, f16);
        for (int e = 0; e < n; ++e) {
            __syncthreads();  // buffer e & 1 is complete; nobody reads the other one any more
            if (e + 1 < n) load(e + 1);
            const int ent = list[e];
            if ((ent >> (12 + hh)) & 1) {
                const int J = ent & 0xfff;
                const int cls = block_class(R0, 32, J * kBC, kBC, g);
                if (cls != kSkip) {
                    f32x16 acc[2][1];
                    O::template scores<1>(acc, kbuf[e & 1], qop);
                    if (cls == kPartial) apply_mask<1>(acc, J, R0, g);
                    // A = [(s - tau)/2]_+^2 with s = scale * (Q.K); A <= 1, so no
                    // partial sum of A V exceeds max |V|
                    if constexpr (GEN) {
#pragma unroll
                        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                            for (int r = 0; r < 16; ++r) {
                                const float sv = acc[kb][0][r] * p.scale;
                                acc[kb][0][r] = wk ? p.am.g(sv, tq) : p.am.p(sv, tq);
                            }
                    } else {
#pragma unroll
                        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                            for (int r = 0; r < 16; ++r) {
                                const float dd = 0.5f * fmaxf(acc[kb][0][r] * p.scale - tq, 0.0f);
                                acc[kb][0][r] = wk ? dd : dd * dd;
                            }
                    }
                    if (wk) {
#pragma unroll
                        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                            for (int r = 0; r < 16; ++r) gs += acc[kb][0][r];
                    }
                    if (f16) {
                        const uint16_t* Vt = vbuf[e & 1];
#pragma unroll
                        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                            for (int s2 = 0; s2 < 2; ++s2) {
                                f16x8 b;
#pragma unroll
                                for (int q = 0; q < 8; ++q) b[q] = (_Float16)acc[kb][0][8 * s2 + q];
#pragma unroll
                                for (int db = 0; db < D / 32; ++db) {
                                    const uint16_t* row = Vt + (db * 32 + m) * kVRow + kb * 32 + 16 * s2 + 4 * h;
                                    const u32x2 lo4 = *reinterpret_cast<const u32x2*>(row);
                                    const u32x2 hi4 = *reinterpret_cast<const u32x2*>(row + 8);
                                    u32x4 vv;
                                    vv[0] = lo4[0]; vv[1] = lo4[1]; vv[2] = hi4[0]; vv[3] = hi4[1];
                                    oa.o[db][0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                                        __builtin_bit_cast(f16x8, vv), b, oa.o[db][0], 0, 0, 0);
                                }
                            }
                    } else {
                        const bool on[2] = {true, true};
                        O::template pv<1>(oa, reinterpret_cast<const __bf16*>(vbuf[e & 1]), acc, on);
                    }
                }
            }
            if (e + 1 < n) over |= store((e + 1) & 1, f16);
        }
        if (over) atomicOr(&vover_s, 1);
        __syncthreads();
    };
    run(true);
    if (vover_s) run(false);  // a V entry beyond fp16 range somewhere in this block's tiles

    // O = sum A V; register r of a lane holds d = db*32 + 8(r/4) + 4h + r%4
    if (wk) gs += __shfl_xor(gs, 32, kWave);
    if (R0 + m < p.L) {
        if (wk && h == 0) p.gsum[(size_t)bh * p.L + R0 + m] = gs;
        float* orow = (wk ? p.gv : p.o) + ((size_t)bh * p.L + R0 + m) * D;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                f32x4 v4;
#pragma unroll
                for (int e = 0; e < 4; ++e) v4[e] = oa.o[db][0][4 * r4 + e];
                *reinterpret_cast<f32x4*>(orow + db * 32 + 8 * r4 + 4 * h) = v4;
            }
    }
}

template <int D, bool GEN>
__global__ __launch_bounds__(kNT, (D == 64 ? 3 : 2)) void fwd_out_bf16_kernel(FwdParams p) {
    __shared__ __attribute__((aligned(16))) OutLds<D> ol;
    __shared__ uint16_t list[kMaxTc];
    __shared__ uint32_t mw[2][kMaxTc / 32];
    __shared__ int nlist_s, vover_s;
    const int t = threadIdx.x;
    int bh, r0;
    decode_item(blockIdx.x, p.BH, p.nQ, p.mode != 0, bh, r0);
    if (p.ostate != nullptr && p.ostate[(size_t)bh * p.nQ + r0 / kBR]) return;  // O already written
    for (int i = t; i < 2 * p.Wd; i += kNT) {
        const int b = i / p.Wd, wd = i % p.Wd;
        const int I = r0 / 64 + b;
        mw[b][wd] = (I < p.Tr64) ? p.mask[((size_t)bh * p.Tr64 + I) * p.Wd + wd] : 0u;
    }
    out_phase_bf16<D, GEN>(p, bh, r0, ol, mw[0], mw[1], list, nlist_s, vover_s, nullptr);
}

// ------------------------------------------------------------ fused, bf16
// The whole forward of a 128-row block in one workgroup: the score
// statistics, the threshold solve, then O (from the candidate lists, or over
// the non-null tiles).  The row statistics, tile maxima, tile lists and mask
// stay in LDS between the phases, the phases' buffers overlap, and Q is read
// once for the first two.  With no O requested (p.o null) it stops after the
// solve.
template <int D, int TCMAX>
struct FusedCfg {
    // three workgroups per CU fit (<= 168 VGPRs, <= 53 KB LDS) at d = 64 with
    // tables for up to 128 key tiles
    static constexpr int kOcc = (D == 64 && TCMAX <= 128) ? 3 : 2;
    // ring stages of the candidate sweeps: two at d = 64 (the next pair of
    // tiles loads while the current one is swept), one at d = 128 (two stages
    // and the solve scratch would not fit beside the second workgroup)
    static constexpr int kSolveS = (D == 64) ? 2 : 1;
};

template <int D, int TCMAX, bool CAUSAL>
__global__ __launch_bounds__(kNT, (FusedCfg<D, TCMAX>::kOcc)) void fwd_fused_kernel(FwdParams p) {
    using T = __bf16;
    using O = Ops<T, D>;
    __shared__ BlockLds<TCMAX> bl;
    union Work {
        T sring[StatsCfg<T, D>::kS * 2 * 64 * D];
        struct {
            T ring[FusedCfg<D, TCMAX>::kSolveS * 2 * 64 * D];
            SolveScratch<true> ss;  // (L <= 16384: a bin count fits 16 bits)
        } solve;
        OutLds<D> out;
    };
    __shared__ __attribute__((aligned(16))) Work wk;
    int bh, r0;
    decode_item(blockIdx.x, p.BH, p.nQ, p.mode != 0, bh, r0);
    {
        typename O::template QOp<2> qop;
        O::load_q(qop, reinterpret_cast<const T*>(p.q) + (size_t)bh * p.L * D, r0 + 64 * (wave_id() & 1), p.L);
        stats_phase<T, D, TCMAX, CAUSAL>(p, bh, r0, qop, wk.sring, bl, true);
        __syncthreads();
        if (solve_phase<T, D, TCMAX, FusedCfg<D, TCMAX>::kSolveS>(p, bh, r0, qop, wk.solve.ring, wk.solve.ss, bl, true))
            return;
    }
    if (p.o == nullptr) return;
    __syncthreads();
    // O, then (when requested) G.V and sum g over the same tiles
    for (int what = 0; what < (p.gv != nullptr ? 2 : 1); ++what) {
        if (what) __syncthreads();
        if (p.gen)
            out_phase_bf16<D, true>(p, bh, r0, wk.out, bl.maskw[0], bl.maskw[1], bl.list, bl.nlist_s, bl.vover_s,
                                    bl.row_tau, what);
        else
            out_phase_bf16<D, false>(p, bh, r0, wk.out, bl.maskw[0], bl.maskw[1], bl.list, bl.nlist_s,
                                     bl.vover_s, bl.row_tau, what);
    }
}

template <typename T, int D, int TCMAX>
void launch_stats(const FwdParams& fp, int grid, hipStream_t stream) {
    if (fp.mode == 1)
        hipLaunchKernelGGL((fwd_stats_kernel<T, D, TCMAX, true>), dim3(grid), dim3(kNT), 0, stream, fp);
    else
        hipLaunchKernelGGL((fwd_stats_kernel<T, D, TCMAX, false>), dim3(grid), dim3(kNT), 0, stream, fp);
}

template <int D, int TCMAX>
void launch_fused(const FwdParams& fp, int grid, hipStream_t stream) {
    if (fp.mode == 1)
        hipLaunchKernelGGL((fwd_fused_kernel<D, TCMAX, true>), dim3(grid), dim3(kNT), 0, stream, fp);
    else
        hipLaunchKernelGGL((fwd_fused_kernel<D, TCMAX, false>), dim3(grid), dim3(kNT), 0, stream, fp);
}

template <typename T, int D>
hipError_t launch_typed(const FwdParams& fp, int grid, int phase, hipStream_t stream) {
    // bf16 threshold (with or without O) up to L = 16384: one fused kernel
    if constexpr (sizeof(T) == 2) {
        if ((phase == 3 || phase == 7) && fp.Tc <= 256) {
            if (fp.Tc <= 128) launch_fused<D, 128>(fp, grid, stream);
            else launch_fused<D, 256>(fp, grid, stream);
            return hipGetLastError();
        }
    }
    if (phase & 1) {
        if (fp.Tc <= 128)
            launch_stats<T, D, 128>(fp, grid, stream);
        else if (fp.Tc <= 256)
            launch_stats<T, D, 256>(fp, grid, stream);
        else
            launch_stats<T, D, kMaxTc>(fp, grid, stream);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (phase & 2) {
        if (fp.Tc <= 128)
            hipLaunchKernelGGL((fwd_solve_kernel<T, D, 128>), dim3(grid), dim3(kNT), 0, stream, fp);
        else if (fp.Tc <= 256)
            hipLaunchKernelGGL((fwd_solve_kernel<T, D, 256>), dim3(grid), dim3(kNT), 0, stream, fp);
        else
            hipLaunchKernelGGL((fwd_solve_kernel<T, D, kMaxTc>), dim3(grid), dim3(kNT), 0, stream, fp);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (phase & 4) {
        if constexpr (sizeof(T) == 2) {
            if (fp.gen)
                hipLaunchKernelGGL((fwd_out_bf16_kernel<D, true>), dim3(grid), dim3(kNT), 0, stream, fp);
            else
                hipLaunchKernelGGL((fwd_out_bf16_kernel<D, false>), dim3(grid), dim3(kNT), 0, stream, fp);
        } else {
            if (fp.gen)
                hipLaunchKernelGGL((fwd_out_kernel<T, D, true>), dim3(grid), dim3(kNT), 0, stream, fp);
            else
                hipLaunchKernelGGL((fwd_out_kernel<T, D, false>), dim3(grid), dim3(kNT), 0, stream, fp);
        }
        return hipGetLastError();
    }
    return hipSuccess;
}

size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t mask_bytes(int B, int H, int L) {
    const size_t tr = (L + 63) / 64, tc = (L + 63) / 64, wd = (tc + 31) / 32;
    return (size_t)B * H * tr * wd * sizeof(uint32_t);
}
size_t rowstat_bytes(int B, int H, int L) { return (size_t)B * H * L * 2 * sizeof(float); }
size_t umax_bytes(int B, int H, int L) {
    const size_t tr = (L + 63) / 64, tc = (L + 63) / 64;
    return (size_t)B * H * tr * tc * sizeof(float);
}
size_t cand_rows(int B, int H, int L) { return (size_t)B * H * ((L + kBR - 1) / kBR) * kBR; }

}  // namespace
}  // namespace attn

size_t attn_threshold_workspace_bytes(int B, int H, int L) {
    using namespace attn;
    const size_t rows = cand_rows(B, H, L);
    return round256(rowstat_bytes(B, H, L)) + round256(umax_bytes(B, H, L)) +
           round256(rows * kCandCap * sizeof(u32x2)) + round256(rows / kBR * sizeof(int));
}

size_t attn_fwd_workspace_bytes(int B, int H, int L, int, int) {
    // threshold scratch, then room for the block mask when the caller does not keep it
    return attn_threshold_workspace_bytes(B, H, L) + attn::round256(attn::mask_bytes(B, H, L));
}

int attn_max_candidate_cap(int, int) { return attn::kCandCap; }

hipError_t launch_attn_fwd(const AttnArgs& a, int phase, hipStream_t stream) {
    using namespace attn;
    if (a.L > kMaxL) return hipErrorInvalidValue;
    FwdParams fp;
    fp.q = a.q; fp.k = a.k; fp.v = a.v; fp.o = a.o; fp.tau = a.tau;
    fp.gv = a.gv; fp.gsum = a.gsum;
    char* ws = reinterpret_cast<char*>(a.workspace);
    fp.rowstat = reinterpret_cast<float*>(ws);
    size_t off = round256(rowstat_bytes(a.B, a.H, a.L));
    fp.umax = reinterpret_cast<float*>(ws + off);
    off += round256(umax_bytes(a.B, a.H, a.L));
    const size_t rows = cand_rows(a.B, a.H, a.L);
    fp.clist = reinterpret_cast<u32x2*>(ws + off);
    off += round256(rows * kCandCap * sizeof(u32x2));
    // the whole forward: the solve kernel writes O from the candidate lists of
    // the blocks it can, and the output kernel skips those blocks
    const bool whole = (phase & 6) == 6;
    fp.ostate = whole ? reinterpret_cast<int*>(ws + off) : nullptr;
    fp.gather = whole ? 1 : 0;
    fp.mask = a.block_mask ? a.block_mask
                           : reinterpret_cast<uint32_t*>(ws + attn_threshold_workspace_bytes(a.B, a.H, a.L));
    fp.BH = a.B * a.H; fp.L = a.L; fp.mode = a.mask;
    fp.W = a.window < a.L ? a.window : a.L;  // a window of L or more is plain causal
    fp.nQ = (a.L + kBR - 1) / kBR;
    fp.Tc = (a.L + kBC - 1) / kBC;
    fp.Tr64 = (a.L + 63) / 64;
    fp.Wd = (fp.Tc + 31) / 32;
    fp.scale = a.scale;
    fp.cap = a.cand_cap;
    fp.am = make_alpha_map(a.alpha);
    fp.gen = a.alpha != 1.5f ? 1 : 0;
    const int grid = fp.nQ * fp.BH;
    if (a.dtype == 1) {
        if (a.d == 64) return launch_typed<__bf16, 64>(fp, grid, phase, stream);
        return launch_typed<__bf16, 128>(fp, grid, phase, stream);
    }
    if (a.d == 64) return launch_typed<float, 64>(fp, grid, phase, stream);
    return launch_typed<float, 128>(fp, grid, phase, stream);
}

}  // namespace entmax
