// attn_fwd.hip -- 1.5-entmax attention forward on gfx950.
//
// Three kernels per call, each one workgroup per 128 query rows of a head:
//
// fwd_stats  one sweep over the tiles the mask mode allows: S^T = K Q^T on
//            MFMA; per row the maximum and the sixteen largest tile maxima
//            (four per lane half and key parity); per (row half, tile) the
//            largest score.  tau_lo = the exact threshold of those tile
//            maxima.  Adding scores to a row only raises its threshold (every
//            term of the normaliser is non-negative), so tau_lo <= tau, and
//            it also clears the bracket end max - 2 of "AdaSplash-2: Faster
//            Differentiable Sparse Attention" sec. 2.4 (score units).
// fwd_solve  collect: over the tiles whose largest score beats tau_lo, every
//            score s > tau_lo is appended to its row's candidate list.
//            Nothing at or below tau_lo can carry weight, so the row's
//            threshold is the threshold of its candidates alone.
//            solve: per row, Newton steps from below on the candidates
//            (f(t) = sum [(s - t)/2]_+^2 - 1 is convex and decreasing) with a
//            bisection guard and an exact finish: once tau lies below the
//            support the normaliser is a quadratic in tau over {s > tau}
//            (S0/S1/S2 of AdaSplash-2 appendix C.3).  Sums are fp64.
//            mask: a 64x64 tile is non-null iff one of its candidates exceeds
//            its row's tau (packed 32 tiles per word, AdaSplash-2 appendix C.4).
//            fallback: rows whose candidates overflow the list are collected
//            again with a tighter bound, then refined by Halley-bisection
//            sweeps over all their tiles, then a sweep marks their tiles.
// fwd_out    walks only the set mask bits of its two 64-row blocks
//            (find-first-set over the packed words, AdaSplash-2 sec. 3.3
//            phase 4), recomputes S, A = [(S - tau)/2]_+^2 and accumulates
//            O = A V on MFMA (bf16 inputs: A and V in fp16, the pages' own
//            casts, with a bf16 hi + lo redo where V leaves the fp16 range).
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
    float* cval;      // workspace [BH * nQ][kCandCap][128]: candidate scores, slot-major per row block
    uint16_t* cjt;    // workspace, same shape: position of each candidate's tile in the tile list
    int BH, L, mode, W, nQ, Tc, Tr64, Wd;
    float scale;
    int cap;
    AlphaMap am;  // the alpha-entmax map
    int gen;      // alpha != 1.5: Newton solves and pow weights
};

// Candidate slots per row in the workspace lists.
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
template <typename T, int D, int S, bool PER_QB = false, class Fn>
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
            if constexpr (PER_QB) {
                // one 32-row block at a time: half the accumulators live, the
                // tile's operands read twice
#pragma unroll
                for (int qb = 0; qb < 2; ++qb) {
                    typename O::template QOp<1> q1;
                    constexpr int kQs = sizeof(q1.q[0]) / sizeof(q1.q[0][0]);
#pragma unroll
                    for (int s = 0; s < kQs; ++s) q1.q[0][s] = qop.q[qb][s];
                    f32x16 acc[2][1];
                    O::template scores<1>(acc, Kt, q1);
                    if (cls == kPartial) apply_mask<1>(acc, J, R0 + 32 * qb, g);
                    fn(J, e, qb, acc);
                }
            } else {
                f32x16 acc[2][2];
                O::scores(acc, Kt, qop);
                if (cls == kPartial) apply_mask(acc, J, R0, g);
                fn(J, e, acc);
            }
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

// Candidate slots per row kept in LDS; further slots live in the workspace.
#ifndef ENTMAX_LDS_CAND
#define ENTMAX_LDS_CAND 48
#endif
constexpr int kLdsCand = ENTMAX_LDS_CAND;

// A row's candidate list: entry i at lds[i * kBR] for i < kLdsCand, else at
// glob[i * kBR] (both slot-major over the 128 rows of a workgroup, so the
// lanes of a wave touch consecutive words).  Two lanes share a row: the lane
// with parity h takes entries start, start + 2, ... (start = h at first).
struct CandSrc {
    const float* lds;
    const float* glob;
    int n, start;
    __device__ __forceinline__ float at(int i) const {
        return i < kLdsCand ? lds[i * kBR] : glob[(size_t)i * kBR];
    }
    template <class F>
    __device__ __forceinline__ void each(F f) const {
        const int nl = n < kLdsCand ? n : kLdsCand;
#pragma unroll 4
        for (int i = start; i < nl; i += 2) f(lds[i * kBR]);
#pragma unroll 4
        for (int i = start > kLdsCand ? start : kLdsCand + (start & 1); i < n; i += 2) f(glob[(size_t)i * kBR]);
    }
};

// The same list with the lane's first KR entries held in registers; missing
// entries read -inf, which no threshold test passes.
template <int KR>
struct RegSrc {
    float v[KR];
    CandSrc tail;  // the lane's entries from start + 2 * KR on
    static_assert(2 * KR <= kLdsCand, "register entries come from LDS");
    __device__ __forceinline__ void load(const CandSrc& src) {
#pragma unroll
        for (int k = 0; k < KR; ++k) {
            const int i = src.start + 2 * k;
            v[k] = (i < src.n) ? src.lds[i * kBR] : neg_inf();
        }
        tail = src;
        tail.start = src.start + 2 * KR;
    }
    template <class F>
    __device__ __forceinline__ void each(F f) const {
#pragma unroll
        for (int k = 0; k < KR; ++k) f(v[k]);
        tail.each(f);
    }
};

// Threshold of a row from its candidates: every entry is above `lo`, and
// none of the row's other scores is.  Two lanes share a row (sums are
// combined with lane l ^ 32).  Newton steps from below: f(t) = sum
// [(x - t)/2]_+^2 - 1 is convex and decreasing, so a step from a point with
// f >= 0 stays at or below the root (bisection takes over if rounding lands
// above it).  Exact finish: when the closed-form root of {x > t} lies below
// the set's smallest member, that set is the support and the root is tau.
// Sums in fp64.  Returns tau; lanes with active == false only take part in
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
            double tn = t + f / F1;
            if (!(tn > lo && tn < hi)) tn = 0.5 * (lo + hi);
            t = tn;
        } else {
            hi = t;
            t = 0.5 * (lo + hi);
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

// Largest entry of a candidate list (two lanes per row).
template <class Src>
__device__ __forceinline__ float list_max(const Src& src) {
    float mx = neg_inf();
    src.each([&](float x) { mx = fmaxf(mx, x); });
    return fmaxf(mx, __shfl_xor(mx, 32, kWave));
}

constexpr int kRounds = 3;  // candidate collections before the sweep fallback

#ifndef ENTMAX_STATS_STAGES_BF16_64
#define ENTMAX_STATS_STAGES_BF16_64 3
#endif
#ifndef ENTMAX_STATS_STAGES_BF16_128
#define ENTMAX_STATS_STAGES_BF16_128 2
#endif
#ifndef ENTMAX_STATS_OCCUPANCY
#define ENTMAX_STATS_OCCUPANCY 3
#endif
// Ring stages (pairs of tiles in flight + 1) of the score-statistics sweep,
// and the number of key tiles per row its on-chip tables are sized for
// (TCMAX * 64 >= L): small tables leave room for three workgroups per CU.
template <typename T, int D>
struct StatsCfg {
    static constexpr int kS = (sizeof(T) == 2 && D == 64) ? ENTMAX_STATS_STAGES_BF16_64
                              : (sizeof(T) == 2) ? ENTMAX_STATS_STAGES_BF16_128
                              : ((D == 128) ? 2 : 3);
};
#ifndef ENTMAX_COLLECT_STAGES
#define ENTMAX_COLLECT_STAGES 2
#endif
#ifndef ENTMAX_COLLECT_OCCUPANCY
#define ENTMAX_COLLECT_OCCUPANCY 2
#endif
// Ring stages and workgroups per CU of the candidate sweep.
#ifndef ENTMAX_COLLECT_STAGES_BF16_128
#define ENTMAX_COLLECT_STAGES_BF16_128 1
#endif
#ifndef ENTMAX_COLLECT_OCCUPANCY_BF16_128
#define ENTMAX_COLLECT_OCCUPANCY_BF16_128 2
#endif
// (bf16, d = 128: a one-stage ring leaves room in LDS for two workgroups per
// CU, whose sweeps then hide each other's loads.)
template <typename T, int D>
struct CollectCfg {
    static constexpr int kS = (sizeof(T) == 4 && D == 128) ? 1
                              : (sizeof(T) == 2 && D == 128) ? ENTMAX_COLLECT_STAGES_BF16_128
                                                             : ENTMAX_COLLECT_STAGES;
    static constexpr int kOcc = (sizeof(T) == 2 && D == 64)    ? ENTMAX_COLLECT_OCCUPANCY
                                : (sizeof(T) == 2 && D == 128) ? ENTMAX_COLLECT_OCCUPANCY_BF16_128
                                                               : 1;
};

#ifndef ENTMAX_COLLECT_PER_QB
#define ENTMAX_COLLECT_PER_QB 0
#endif
// The candidate sweeps take one 32-row block at a time (fewer live
// accumulators, each tile's operands read twice) where that lets the kernel
// keep more workgroups per CU.
template <typename T, int D>
constexpr bool kCollectPerQb = sizeof(T) == 2 && D == 64 && ENTMAX_COLLECT_PER_QB;

constexpr int kTop4 = 4;  // tile maxima kept per lane half per row

// ------------------------------------------------------------ kernel 1a
// Dense sweep: per row the top tile maxima (-> tau_lo and the maximum) and
// per (64-row half, tile) the largest raw score.
// CAUSAL: the instance for the causal mask (its list-free sweep covers the
// tiles up to the diagonal); the other serves no mask and the window mask
// (which always takes the list).  Separate instances keep each loop's code
// as it is alone.
template <typename T, int D, int TCMAX, bool CAUSAL>
__global__ __launch_bounds__(kNT, ENTMAX_STATS_OCCUPANCY) void fwd_stats_kernel(FwdParams p) {
    using O = Ops<T, D>;
    constexpr int S = StatsCfg<T, D>::kS;
    __shared__ __attribute__((aligned(16))) T ring[S * 2 * 64 * D];
    __shared__ uint16_t list[TCMAX];
    __shared__ float umax[2][TCMAX];
    __shared__ int nlist_s;
    // the per-row lists are merged through the ring once the sweep is over
    typedef float StRow[kBR][2 * kTop4];
    static_assert(sizeof(float) * 2 * kBR * 2 * kTop4 <= sizeof(T) * S * 2 * 64 * D, "merge space");
    StRow* st = reinterpret_cast<StRow*>(ring);

    const int t = threadIdx.x, w = wave_id(), qh = w & 1, kh = w >> 1;
    const int l = lane_id(), m = l & 31, h = l >> 5;
    int bh, r0;
    decode_item(blockIdx.x, p.BH, p.nQ, p.mode != 0, bh, r0);
    const int R0 = r0 + 64 * qh;
    const Geom g = {p.L, p.mode, p.W};
    const size_t head_off = (size_t)bh * p.L * D;
    const T* Qh = reinterpret_cast<const T*>(p.q) + head_off;
    const T* Kh = reinterpret_cast<const T*>(p.k) + head_off;

    typename O::template QOp<2> qop;
    O::load_q(qop, Qh, R0, p.L);
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
    }
    for (int i = t; i < 2 * p.Tc; i += kNT) {
        const int hh = i / p.Tc, J = i % p.Tc;
        const int I = r0 / 64 + hh;
        if (I < p.Tr64) p.umax[((size_t)bh * p.Tr64 + I) * p.Tc + J] = umax[hh][J];
    }
}

// ------------------------------------------------------------ kernel 1b
// Candidate sweep over the tiles whose best score beats tau_lo: every score
// above its row's tau_lo goes to the row's list (global memory, so the
// workgroup's LDS stays small).  Rows whose list overflows get a tighter
// bound (the threshold of the candidates they kept, a lower bound on tau
// since tau only grows with the set) and are collected again; rows still
// overflowing after kRounds are solved by Halley-bisection sweeps.  Then the
// exact tau of every complete list (two lanes per row, the first
// 2 * kSolveRegs<D> candidates in registers), its non-null tiles (those holding
// a candidate above tau), and tau and the mask words of both 64-row blocks.
#ifndef ENTMAX_SOLVE_REGS
#define ENTMAX_SOLVE_REGS 16
#endif
#ifndef ENTMAX_SOLVE_REGS_128
#define ENTMAX_SOLVE_REGS_128 8
#endif
// (d = 128 keeps fewer candidates in registers: its query operand takes twice
// the registers, and the kernel runs two workgroups per CU.)
template <int D>
constexpr int kSolveRegs = D == 128 ? ENTMAX_SOLVE_REGS_128 : ENTMAX_SOLVE_REGS;

template <typename T, int D, int TCMAX>
__global__ __launch_bounds__(kNT, (CollectCfg<T, D>::kOcc)) void fwd_solve_kernel(FwdParams p) {
    using O = Ops<T, D>;
    constexpr int S = CollectCfg<T, D>::kS;
    constexpr int WD = TCMAX / 32;
    __shared__ __attribute__((aligned(16))) T ring[S * 2 * 64 * D];
    // candidate slots [slot][row], then one spare word per thread
    __shared__ float lval[kLdsCand * kBR + kNT];
    __shared__ uint16_t lpos[kLdsCand * kBR + kNT];
    __shared__ uint16_t list[TCMAX];
    __shared__ float um_s[2][TCMAX];
    __shared__ int cnt[kBR], rstate[kBR];
    __shared__ float row_m[kBR], row_lo[kBR], row_hi[kBR], row_tau[kBR];
    __shared__ uint32_t maskw[2][WD];
    __shared__ int nlist_s, flag_s;

    const int t = threadIdx.x, w = wave_id(), qh = w & 1, kh = w >> 1;
    const int l = lane_id(), m = l & 31, h = l >> 5;
    int bh, r0;
    decode_item(blockIdx.x, p.BH, p.nQ, p.mode != 0, bh, r0);
    const size_t blk = (size_t)bh * p.nQ + r0 / kBR;
    const int R0 = r0 + 64 * qh;
    const Geom g = {p.L, p.mode, p.W};
    const size_t head_off = (size_t)bh * p.L * D;
    const T* Qh = reinterpret_cast<const T*>(p.q) + head_off;
    const T* Kh = reinterpret_cast<const T*>(p.k) + head_off;
    const int cap = p.cap < kCandCap ? p.cap : kCandCap;
    float* cval = p.cval + blk * kCandCap * kBR;
    uint16_t* cjt = p.cjt + blk * kCandCap * kBR;
    const float2* rowstat = reinterpret_cast<const float2*>(p.rowstat) + (size_t)bh * p.L;

    typename O::template QOp<2> qop;
    O::load_q(qop, Qh, R0, p.L);
    // row statistics and the tile maxima of both row blocks, loaded together
    if (t < kBR) {
        const bool valid = (r0 + t) < p.L;
        const float2 rs = valid ? rowstat[r0 + t] : make_float2(neg_inf(), __builtin_inff());
        row_m[t] = rs.x;
        row_lo[t] = rs.y;
        cnt[t] = 0;
        rstate[t] = valid ? 1 : 0;  // 1: to collect, 3: list complete, 2: sweep fallback, 0: no row
    }
    for (int i = t; i < 2 * p.Tc; i += kNT) {
        const int hh = i / p.Tc, J = i - hh * p.Tc;
        const int I = r0 / 64 + hh;
        um_s[hh][J] = (I < p.Tr64) ? p.umax[((size_t)bh * p.Tr64 + I) * p.Tc + J] * p.scale : neg_inf();
    }
    for (int i = t; i < 2 * WD; i += kNT) (&maskw[0][0])[i] = 0u;
    __syncthreads();

    // tiles whose best score beats the smallest tau_lo of the row half
    if (w == 0) {
        const float th0 = wave_min(row_lo[l]), th1 = wave_min(row_lo[64 + l]);
        const int n = build_list(list, p.Tc, [&](int J) {
            return (um_s[0][J] > th0 ? 1 : 0) | (um_s[1][J] > th1 ? 2 : 0);
        });
        if (l == 0) nlist_s = n;
    }
    __syncthreads();

    const int srow = qh * 64 + kh * 32 + m;  // the row this lane handles (with lane l ^ 32)
    const int lds_lim = cap < kLdsCand ? cap : kLdsCand;
    const int spare = kLdsCand * kBR + t;
    for (int round = 0; round < kRounds; ++round) {
        float lo_q[2];
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            const int row = qh * 64 + qb * 32 + m;
            lo_q[qb] = rstate[row] == 1 ? row_lo[row] : __builtin_inff();
        }
        // the candidates of one 32-row block (column c of acc) of list entry e
        auto collect_qb = [&](int e, int qb, auto& acc, int c) {
            float bm = neg_inf();
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) bm = fmaxf(bm, acc[kb][c][r]);
            if (__ballot(bm * p.scale > lo_q[qb]) == 0) return;
            const float lo = lo_q[qb];
            int nb = 0;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    acc[kb][c][r] *= p.scale;
                    nb += acc[kb][c][r] > lo ? 1 : 0;
                }
            const int row = qh * 64 + qb * 32 + m;
            int base = 0;
            if (nb) base = atomicAdd(&cnt[row], nb);
            if (__ballot(base + nb > lds_lim) == 0) {
                // all in LDS: the lane's candidates take consecutive slots from
                // base in register order; other elements write the spare word
                int slot = base;
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const bool on = acc[kb][c][r] > lo;
                        const int a = on ? slot * kBR + row : spare;
                        lval[a] = acc[kb][c][r];
                        lpos[a] = (uint16_t)e;
                        slot += on ? 1 : 0;
                    }
            } else {
                // the list spills past LDS: candidates in register order from
                // base, LDS slots first, then the workspace, the rest dropped
                // (the row is then collected again with a tighter bound)
                int slot = base;
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const float sv = acc[kb][c][r];
                        if (sv > lo) {
                            if (slot < lds_lim) {
                                lval[slot * kBR + row] = sv;
                                lpos[slot * kBR + row] = (uint16_t)e;
                            } else if (slot < cap) {
                                cval[(size_t)slot * kBR + row] = sv;
                                cjt[(size_t)slot * kBR + row] = (uint16_t)e;
                            }
                            ++slot;
                        }
                    }
            }
        };
        if constexpr (kCollectPerQb<T, D>) {
            ring_sweep<T, D, S, true>(list, nlist_s, Kh, ring, qop, R0, g,
                                      [&](int, int e, int qb, f32x16(&acc)[2][1]) { collect_qb(e, qb, acc, 0); });
        } else {
            ring_sweep<T, D, S>(list, nlist_s, Kh, ring, qop, R0, g, [&](int, int e, f32x16(&acc)[2][2]) {
#pragma unroll
                for (int qb = 0; qb < 2; ++qb) collect_qb(e, qb, acc, qb);
            });
        }

        const bool open = rstate[srow] == 1;
        const int nc = cnt[srow];
        const bool over = open && nc > cap;
        float lo_new = neg_inf();
        if (__ballot(over) != 0) {
            // threshold of the kept candidates: a lower bound on the row's tau
            const CandSrc src = {lval + srow, cval + srow, over ? cap : 0, h};
            const float smax = list_max(src);
            if (p.gen) {
                float lb;
                solve_candidates_gen(src, smax - p.am.e, p.am.hi(smax, (float)cap), over, p.am, &lb);
                lo_new = lb - 1e-6f * fmaxf(1.0f, fabsf(lb));
            } else {
                const double ts = solve_candidates(src, smax, (double)smax - 2.0,
                                                   (double)smax - 2.0 / sqrt((double)cap), over);
                lo_new = __double2float_rd(ts);
            }
        }
        if (h == 0 && open) {
            if (!over) {
                rstate[srow] = 3;  // list complete, nc entries
            } else {
                // every score above tau is above lo, so at most nc of them
                row_hi[srow] = p.gen ? p.am.hi(row_m[srow], (float)nc)
                                     : (float)((double)row_m[srow] - 2.0 / sqrt((double)nc));
                const float nl = fmaxf(row_lo[srow], lo_new);
                if (round == kRounds - 1 || !(nl > row_lo[srow])) rstate[srow] = 2;
                row_lo[srow] = nl;
                cnt[srow] = 0;
            }
        }
        if (t == 0) flag_s = 0;
        __syncthreads();
        if (h == 0 && rstate[srow] == 1) atomicOr(&flag_s, 1);
        __syncthreads();
        if (!flag_s) break;
    }

    if (t == 0) flag_s = 0;
    __syncthreads();
    if (h == 0 && rstate[srow] == 2) atomicOr(&flag_s, 1);
    __syncthreads();

    // ---- fallback: Halley-bisection sweeps for rows whose list overflowed
    if (flag_s) {
        __shared__ float fb_t[kBR];
        __shared__ int fb_active[kBR];
        __shared__ float fb_part[kBR][2][3];
        if (h == 0) {
            fb_active[srow] = rstate[srow] == 2 ? 1 : 0;
            fb_t[srow] = row_lo[srow];
        }
        __syncthreads();
        for (int it = 0; it < kFbMaxIter; ++it) {
            float tq[2];
            bool aq[2];
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
                const int row = qh * 64 + qb * 32 + m;
                aq[qb] = fb_active[row] != 0;
                tq[qb] = fb_t[row];
            }
            float sc[2] = {0.f, 0.f}, sf[2] = {0.f, 0.f}, sf1[2] = {0.f, 0.f};
            // this lane's sums over the scores above tq of 32-row block qb
            auto sums_qb = [&](int qb, auto& acc, int c) {
                if (!aq[qb]) return;
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const float s = acc[kb][c][r] * p.scale;
                        if (s > tq[qb]) {
                            sc[qb] += 1.f;
                            if (p.gen) {
                                // F = sum p, F1 = sum p/u (Newton)
                                const float u = p.am.am1 * (s - tq[qb]);
                                const float q = p.am.pw1(u);  // p / u
                                sf[qb] = fmaf(q, u, sf[qb]);
                                sf1[qb] += q;
                            } else {
                                const float gg = 0.5f * (s - tq[qb]);
                                sf[qb] += gg * gg;
                                sf1[qb] += gg;
                            }
                        }
                    }
            };
            if constexpr (kCollectPerQb<T, D>) {
                ring_sweep<T, D, S, true>(list, nlist_s, Kh, ring, qop, R0, g,
                                          [&](int, int, int qb, f32x16(&acc)[2][1]) { sums_qb(qb, acc, 0); });
            } else {
                ring_sweep<T, D, S>(list, nlist_s, Kh, ring, qop, R0, g, [&](int, int, f32x16(&acc)[2][2]) {
#pragma unroll
                    for (int qb = 0; qb < 2; ++qb) sums_qb(qb, acc, qb);
                });
            }
            // combine the two lane halves, then the two key parities
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
                sc[qb] += __shfl_xor(sc[qb], 32, kWave);
                sf[qb] += __shfl_xor(sf[qb], 32, kWave);
                sf1[qb] += __shfl_xor(sf1[qb], 32, kWave);
                if (h == 0) {
                    const int row = qh * 64 + qb * 32 + m;
                    fb_part[row][kh][0] = sc[qb];
                    fb_part[row][kh][1] = sf[qb];
                    fb_part[row][kh][2] = sf1[qb];
                }
            }
            if (t == 0) flag_s = 0;
            __syncthreads();
            if (h == 0 && fb_active[srow]) {
                const float C = fb_part[srow][0][0] + fb_part[srow][1][0];
                const float F = fb_part[srow][0][1] + fb_part[srow][1][1];
                const float F1 = fb_part[srow][0][2] + fb_part[srow][1][2];
                float lo = row_lo[srow], hi = row_hi[srow], tc = fb_t[srow];
                if (p.gen) {
                    bool fin;
                    const float tn = newton_or_bisect(tc, F, F1, lo, hi, &fin, p.am);
                    if (fin || hi - lo <= 4e-7f * fmaxf(1.0f, fabsf(tc))) {
                        fb_active[srow] = 0;
                        row_tau[srow] = fin ? tn : 0.5f * (lo + hi);
                    } else {
                        fb_t[srow] = tn;
                        atomicOr(&flag_s, 1);
                    }
                } else {
                    if (F - 1.0f >= 0.0f) lo = tc; else hi = tc;
                    if (hi - lo <= 4e-7f * fmaxf(1.0f, fabsf(tc))) {
                        fb_active[srow] = 0;
                        row_tau[srow] = 0.5f * (lo + hi);
                    } else {
                        fb_t[srow] = halley_or_bisect(tc, F, F1, C, lo, hi);
                        atomicOr(&flag_s, 1);
                    }
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
        // mark the tiles of the fallback rows
        float tq[2];
        bool aq[2];
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            const int row = qh * 64 + qb * 32 + m;
            aq[qb] = rstate[row] == 2;
            tq[qb] = row_tau[row];
        }
        // set the tile's bit if a score of an active row of block qb is above its tau
        auto mark_qb = [&](int J, int qb, auto& acc, int c) {
            bool any = false;
            if (aq[qb]) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) any |= acc[kb][c][r] * p.scale > tq[qb];
            }
            return any;
        };
        if constexpr (kCollectPerQb<T, D>) {
            ring_sweep<T, D, S, true>(list, nlist_s, Kh, ring, qop, R0, g, [&](int J, int, int qb, f32x16(&acc)[2][1]) {
                if (__ballot(mark_qb(J, qb, acc, 0)) != 0 && l == 0) atomicOr(&maskw[qh][J >> 5], 1u << (J & 31));
            });
        } else {
            ring_sweep<T, D, S>(list, nlist_s, Kh, ring, qop, R0, g, [&](int J, int, f32x16(&acc)[2][2]) {
                bool any = false;
#pragma unroll
                for (int qb = 0; qb < 2; ++qb) any |= mark_qb(J, qb, acc, qb);
                if (__ballot(any) != 0 && l == 0) atomicOr(&maskw[qh][J >> 5], 1u << (J & 31));
            });
        }
    }

    // ---- exact tau of the rows with complete lists
    {
        const bool act = rstate[srow] == 3;
        const int n = act ? cnt[srow] : 0;
        RegSrc<kSolveRegs<D>> src;
        src.load(CandSrc{lval + srow, cval + srow, n, h});
        const double mx = row_m[srow];
        const float tr = p.gen ? solve_candidates_gen(src, row_lo[srow], p.am.hi(row_m[srow], (float)(n > 0 ? n : 1)),
                                                      act, p.am)
                               : (float)solve_candidates(src, mx, row_lo[srow],
                                                         mx - 2.0 / sqrt((double)(n > 0 ? n : 1)), act);
        const int nl = nlist_s;
        auto pos_of = [&](int i) -> int {
            return i < kLdsCand ? lpos[i * kBR + srow] : cjt[(size_t)i * kBR + srow];
        };
        if (nl <= 64) {
            // list positions holding a support entry, OR-ed over the wave, then
            // one lane per position sets the tile's bit
            uint64_t lm = 0;
            if (act) {
#pragma unroll
                for (int k = 0; k < kSolveRegs<D>; ++k) {
                    const uint64_t b = 1ull << (pos_of(h + 2 * k) & 63);
                    lm |= (src.v[k] > tr) ? b : 0ull;
                }
                for (int i = h + 2 * kSolveRegs<D>; i < n; i += 2)
                    if (src.tail.at(i) > tr) lm |= 1ull << pos_of(i);
            }
            const uint32_t lo32 = wave_or((uint32_t)lm), hi32 = wave_or((uint32_t)(lm >> 32));
            const uint32_t mine = (l < 32) ? (lo32 >> l) & 1u : (hi32 >> (l - 32)) & 1u;
            if (l < nl && mine) {
                const int J = list[l] & 0xfff;
                atomicOr(&maskw[qh][J >> 5], 1u << (J & 31));
            }
        } else if (act) {
            for (int i = h; i < n; i += 2)
                if (src.tail.at(i) > tr) {
                    const int J = list[pos_of(i)] & 0xfff;
                    atomicOr(&maskw[qh][J >> 5], 1u << (J & 31));
                }
        }
        if (act && h == 0) row_tau[srow] = tr;
    }
    __syncthreads();

    // ---- outputs: tau and the packed mask of both 64-row blocks
    if (t < kBR && r0 + t < p.L) p.tau[(size_t)bh * p.L + r0 + t] = row_tau[t];
    for (int i = t; i < 2 * p.Wd; i += kNT) {
        const int hh = i / p.Wd, wd = i % p.Wd;
        const int I = r0 / 64 + hh;
        if (I < p.Tr64) p.mask[((size_t)bh * p.Tr64 + I) * p.Wd + wd] = maskw[hh][wd];
    }
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
template <int D, bool GEN>
__global__ __launch_bounds__(kNT, (D == 64 ? 3 : 2)) void fwd_out_bf16_kernel(FwdParams p) {
    using O = Ops<__bf16, D>;
    constexpr int kVRow = O::kVRow;
    constexpr int kKPer = O::kChunks / kNT;  // K chunks per thread per tile
    static_assert(O::kChunks % kNT == 0 && O::kVUnits <= kNT, "staging split");
    __shared__ __attribute__((aligned(16))) __bf16 kbuf[2][O::kKTile];
    __shared__ __attribute__((aligned(16))) uint16_t vbuf[2][D * kVRow];  // fp16 or bf16 bits
    __shared__ uint16_t list[kMaxTc];
    __shared__ uint32_t mw[2][kMaxTc / 32];
    __shared__ int nlist_s, vover_s;

    const int t = threadIdx.x, w = wave_id();
    const int l = lane_id(), m = l & 31, h = l >> 5;
    int bh, r0;
    decode_item(blockIdx.x, p.BH, p.nQ, p.mode != 0, bh, r0);
    const int R0 = r0 + 32 * w;  // this wave's rows
    const int hh = w >> 1;       // their 64-row block
    const Geom g = {p.L, p.mode, p.W};
    const size_t head_off = (size_t)bh * p.L * D;
    const __bf16* Qh = reinterpret_cast<const __bf16*>(p.q) + head_off;
    const __bf16* Kh = reinterpret_cast<const __bf16*>(p.k) + head_off;
    const __bf16* Vh = reinterpret_cast<const __bf16*>(p.v) + head_off;

    for (int i = t; i < 2 * p.Wd; i += kNT) {
        const int b = i / p.Wd, wd = i % p.Wd;
        const int I = r0 / 64 + b;
        mw[b][wd] = (I < p.Tr64) ? p.mask[((size_t)bh * p.Tr64 + I) * p.Wd + wd] : 0u;
    }
    if (t == 0) vover_s = 0;
    __syncthreads();
    if (w == 0) {
        const int n = build_list(list, p.Tc, [&](int J) {
            return (int)((mw[0][J >> 5] >> (J & 31)) & 1u) | (int)(((mw[1][J >> 5] >> (J & 31)) & 1u) << 1);
        });
        if (l == 0) nlist_s = n;
    }
    typename O::template QOp<1> qop;
    O::load_q(qop, Qh, R0, p.L);
    const float tq = (R0 + m < p.L) ? p.tau[(size_t)bh * p.L + R0 + m] : __builtin_inff();
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
    auto run = [&](bool f16) {
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
                            for (int r = 0; r < 16; ++r) acc[kb][0][r] = p.am.p(acc[kb][0][r] * p.scale, tq);
                    } else {
#pragma unroll
                        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                            for (int r = 0; r < 16; ++r) {
                                const float dd = 0.5f * fmaxf(acc[kb][0][r] * p.scale - tq, 0.0f);
                                acc[kb][0][r] = dd * dd;
                            }
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
    if (R0 + m < p.L) {
        float* orow = p.o + ((size_t)bh * p.L + R0 + m) * D;
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

template <typename T, int D, int TCMAX>
void launch_stats(const FwdParams& fp, int grid, hipStream_t stream) {
    if (fp.mode == 1)
        hipLaunchKernelGGL((fwd_stats_kernel<T, D, TCMAX, true>), dim3(grid), dim3(kNT), 0, stream, fp);
    else
        hipLaunchKernelGGL((fwd_stats_kernel<T, D, TCMAX, false>), dim3(grid), dim3(kNT), 0, stream, fp);
}

template <typename T, int D>
hipError_t launch_typed(const FwdParams& fp, int grid, int phase, hipStream_t stream) {
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
           round256(rows * kCandCap * sizeof(float)) + round256(rows * kCandCap * sizeof(uint16_t));
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
    char* ws = reinterpret_cast<char*>(a.workspace);
    fp.rowstat = reinterpret_cast<float*>(ws);
    size_t off = round256(rowstat_bytes(a.B, a.H, a.L));
    fp.umax = reinterpret_cast<float*>(ws + off);
    off += round256(umax_bytes(a.B, a.H, a.L));
    const size_t rows = cand_rows(a.B, a.H, a.L);
    fp.cval = reinterpret_cast<float*>(ws + off);
    off += round256(rows * kCandCap * sizeof(float));
    fp.cjt = reinterpret_cast<uint16_t*>(ws + off);
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
