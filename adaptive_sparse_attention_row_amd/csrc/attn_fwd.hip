// attn_fwd.hip -- 1.5-entmax attention forward on gfx950.
//
// Two kernels per call, both one workgroup per 128 query rows of a head:
//
// fwd_tau  (threshold and block mask)
//   sweep 1  over the tiles the mask mode allows: S^T = K Q^T on MFMA; per
//            row the maximum and the eight largest tile maxima; per (row
//            half, tile) the largest score.
//   bound    tau_lo = the exact threshold of those tile maxima.  Adding
//            scores to a row only raises its threshold (every term of the
//            normaliser is non-negative), so tau_lo <= tau, and it also
//            clears the bracket end max - 2 of "AdaSplash-2: Faster
//            Differentiable Sparse Attention" sec. 2.4 (score units).
//   sweep 2  over the tiles whose largest score beats tau_lo: every score
//            s > tau_lo is appended to its row's candidate list in LDS.
//            Nothing at or below tau_lo can carry weight, so the row's
//            threshold is the threshold of its candidates alone.
//   solve    per row, Halley-bisection on the candidates (the hybrid solver
//            of "AdaSplash: Adaptive Sparse Flash Attention", summary,
//            Approach) with an exact finish: once tau lies below the support
//            the normaliser is a quadratic in tau over {s > tau} (S0/S1/S2 of
//            AdaSplash-2 appendix C.3).  Sums are fp64.
//   mask     a 64x64 tile is non-null iff one of its candidates exceeds its
//            row's tau (packed 32 tiles per word, AdaSplash-2 appendix C.4).
//   fallback rows whose candidates overflow the list are refined by
//            Halley-bisection sweeps over all their tiles, then a sweep
//            marks their tiles.
// fwd_out  (output)
//   walks only the set mask bits of its two 64-row blocks (find-first-set
//   over the packed words, AdaSplash-2 sec. 3.3 phase 4), recomputes S,
//   A = [(S - tau)/2]_+^2 and accumulates O = A V on MFMA (A split into bf16
//   hi + lo so the product keeps ~16 bits of A).
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
    int BH, L, mode, W, nQ, Tc, Tr64, Wd;
    float scale;
    int cap;
};

// Candidate capacity per row (LDS-limited) and K buffering per variant.
template <typename T, int D>
struct FwdCfg {
    static constexpr int kCap = (sizeof(T) == 2 && D == 64) ? 128 : 96;
    static constexpr int kNBuf = (sizeof(T) == 4 && D == 128) ? 1 : 2;
};

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
    const int t = threadIdx.x, w = t / kWave, qh = w & 1, kh = w >> 1;
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
// flight, and call fn(J, cls, acc) for every tile flagged for this wave's row
// half.  One barrier per pair; the global loads stay outstanding across it.
template <typename T, int D, int S, class Fn>
__device__ __forceinline__ void ring_sweep(const uint16_t* list, int n, const T* Kh, T* ring,
                                           const typename Ops<T, D>::template QOp<2>& qop, int R0,
                                           const Geom& g, Fn fn) {
    using O = Ops<T, D>;
    using DMA = TileDMA<T, D>;
    constexpr int kIpp = DMA::template instrs<2>();
    constexpr int kStage = 2 * DMA::kTileElems;
    const int w = threadIdx.x / kWave, qh = w & 1, kh = w >> 1;
    const int npairs = (n + 1) / 2;
    if (npairs == 0) return;
    const auto ln = DMA::template lanes<2>();
    auto issue = [&](int pp) {
        int r0[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int e = 2 * pp + u;
            r0[u] = (e < n) ? (list[e] & 0xfff) * kBC : 0;
        }
        DMA::template issue<2>(ring + (pp % S) * kStage, Kh, r0, g.L, ln);
    };
#pragma unroll
    for (int pp = 0; pp < S - 1; ++pp)
        if (pp < npairs) issue(pp);
    for (int pp = 0; pp < npairs; ++pp) {
        if constexpr (S == 1) {
            // single stage: wait for the previous tile's readers, then load
            barrier_keep_vm();
            issue(pp);
            wait_vmcnt<0>();
        } else {
            if (npairs - 1 - pp >= S - 2) wait_vmcnt<(S - 2) * kIpp>();
            else wait_vmcnt<0>();
        }
        barrier_keep_vm();
        if (S > 1 && pp + S - 1 < npairs) issue(pp + S - 1);
        const int e = 2 * pp + kh;
        if (e < n) {
            const int ent = list[e];
            const int J = ent & 0xfff;
            if ((ent >> (12 + qh)) & 1) {
                const int cls = tile_class(J, R0, g);
                if (cls != kSkip) {
                    f32x16 acc[2][2];
                    O::scores(acc, ring + (pp % S) * kStage + kh * DMA::kTileElems, qop);
                    if (cls == kPartial) apply_mask(acc, J, R0, g);
                    fn(J, cls, acc);
                }
            }
        }
    }
    __syncthreads();
}

// Maximum over the 64 lanes of a wave, by DPP row shifts and broadcasts
// (VALU only), returned to every lane.
__device__ __forceinline__ float wave_max_dpp(float x) {
// lanes without a source read -inf (the identity of max), so no copy of x
// is needed per step
#define ENTMAX_DPP_MAX(ctrl, rmask)                                                              \
    x = fmaxf(x, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(                          \
                     __builtin_bit_cast(int, neg_inf()), __builtin_bit_cast(int, x), ctrl, rmask, \
                     0xf, false)))
    ENTMAX_DPP_MAX(0x111, 0xf);  // row_shr:1
    ENTMAX_DPP_MAX(0x112, 0xf);  // row_shr:2
    ENTMAX_DPP_MAX(0x114, 0xf);  // row_shr:4
    ENTMAX_DPP_MAX(0x118, 0xf);  // row_shr:8  -> lane 15 of each row holds the row max
    ENTMAX_DPP_MAX(0x142, 0xa);  // row_bcast:15
    ENTMAX_DPP_MAX(0x143, 0xc);  // row_bcast:31 -> lane 63 holds the wave max
#undef ENTMAX_DPP_MAX
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 63));
}

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

// Threshold of a row from its candidate list cv[0..n): every entry is above
// `lo`, and none of the row's other scores is.  Two lanes share a row (h = 0
// and 1 take alternate entries; sums are combined with lane l ^ 32).
// Newton steps from below: f(t) = sum [(x - t)/2]_+^2 - 1 is convex and
// decreasing, so a step from a point with f >= 0 stays at or below the root
// (bisection takes over if rounding lands above it).  Exact finish: when the
// closed-form root of {x > t} lies below the set's smallest member, that set
// is the support and the root is tau.  Sums in fp64.  Returns tau; lanes with
// active == false only take part in the exchanges.
__device__ double solve_candidates(const float* cv, int n, double mx, double lo, double hi,
                                   bool active, int h) {
    double t = lo, result = lo;
    bool done = !active;
    for (int it = 0; it < kMaxIter; ++it) {
        if (__ballot(!done) == 0) break;
        double C = 0, S1 = 0, S2 = 0, F = 0, F1 = 0;
        float mn = __builtin_inff();
        if (!done) {
            for (int i = h; i < n; i += 2) {
                const float x = cv[i];
                if ((double)x > t) {
                    const double y = (double)x - mx;
                    const double gg = 0.5 * ((double)x - t);
                    C += 1.0; S1 += y; S2 += y * y; F += gg * gg; F1 += gg;
                    mn = fminf(mn, x);
                }
            }
        }
        C += __shfl_xor(C, 32, kWave);
        S1 += __shfl_xor(S1, 32, kWave);
        S2 += __shfl_xor(S2, 32, kWave);
        F += __shfl_xor(F, 32, kWave);
        F1 += __shfl_xor(F1, 32, kWave);
        mn = fminf(mn, __shfl_xor(mn, 32, kWave));
        if (done) continue;
        const double f = F - 1.0;
        if (f >= 0.0 && C > 0.0) {
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

// Largest entry of a candidate list (two lanes per row).
__device__ __forceinline__ float list_max(const float* cv, int n, int h) {
    float mx = neg_inf();
    for (int i = h; i < n; i += 2) mx = fmaxf(mx, cv[i]);
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
template <typename T, int D>
struct SolveCfg {
    static constexpr int kS = (sizeof(T) == 2 && D == 64) ? 3 : ((sizeof(T) == 4 && D == 128) ? 1 : 2);
};

constexpr int kTop4 = 4;  // tile maxima kept per lane half per row

// ------------------------------------------------------------ kernel 1a
// Dense sweep: per row the top tile maxima (-> tau_lo and the maximum) and
// per (64-row half, tile) the largest raw score.
template <typename T, int D, int TCMAX>
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

    const int t = threadIdx.x, w = t / kWave, qh = w & 1, kh = w >> 1;
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
    if (w == 0) {
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

    ring_sweep<T, D, S>(list, nlist_s, Kh, ring, qop, R0, g, [&](int J, int, f32x16(&acc)[2][2]) {
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
    });

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
        const float lo = tau_of_sorted(v);
        reinterpret_cast<float2*>(p.rowstat)[(size_t)bh * p.L + grow] = make_float2(v[0], lo);
    }
    for (int i = t; i < 2 * p.Tc; i += kNT) {
        const int hh = i / p.Tc, J = i % p.Tc;
        const int I = r0 / 64 + hh;
        if (I < p.Tr64) p.umax[((size_t)bh * p.Tr64 + I) * p.Tc + J] = umax[hh][J];
    }
}

// ------------------------------------------------------------ kernel 1b
// Candidate sweep, exact per-row tau, block mask, fallback.
template <typename T, int D>
__global__ __launch_bounds__(kNT, 1) void fwd_solve_kernel(FwdParams p) {
    using O = Ops<T, D>;
    constexpr int CAP = FwdCfg<T, D>::kCap;
    constexpr int S = SolveCfg<T, D>::kS;

    __shared__ __attribute__((aligned(16))) T ring[S * 2 * 64 * D];
    // odd row stride: the lanes of a wave read the same slot of 32 different
    // rows at once, which must fall in different banks
    constexpr int CST = CAP + 1;
    __shared__ __attribute__((aligned(16))) float cval[kBR * CST];
    __shared__ uint16_t cjt[kBR * CST];
    __shared__ uint16_t list[kMaxTc];
    __shared__ int cnt[kBR];
    __shared__ float row_m[kBR], row_lo[kBR], row_tau[kBR];
    __shared__ uint32_t maskw[2][kMaxTc / 32];
    __shared__ int nlist_s, ovf_s;
    __shared__ float fb_part[kBR][2][3];

    const int t = threadIdx.x, w = t / kWave, qh = w & 1, kh = w >> 1;
    const int l = lane_id(), m = l & 31, h = l >> 5;
    int bh, r0;
    decode_item(blockIdx.x, p.BH, p.nQ, p.mode != 0, bh, r0);
    const int R0 = r0 + 64 * qh;
    const Geom g = {p.L, p.mode, p.W};
    const size_t head_off = (size_t)bh * p.L * D;
    const T* Qh = reinterpret_cast<const T*>(p.q) + head_off;
    const T* Kh = reinterpret_cast<const T*>(p.k) + head_off;
    const int cap = p.cap < CAP ? p.cap : CAP;

    typename O::template QOp<2> qop;
    O::load_q(qop, Qh, R0, p.L);
    if (t < kBR) {
        const int grow = r0 + t;
        float2 rs = make_float2(neg_inf(), __builtin_inff());
        if (grow < p.L) rs = reinterpret_cast<const float2*>(p.rowstat)[(size_t)bh * p.L + grow];
        row_m[t] = rs.x;
        row_lo[t] = rs.y;
        cnt[t] = 0;
    }
    for (int i = t; i < 2 * (kMaxTc / 32); i += kNT) (&maskw[0][0])[i] = 0u;
    __syncthreads();

    // tiles whose best score beats the smallest tau_lo of the row half
    if (w == 0) {
        float th[2];
        const float* um[2];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            th[hh] = wave_min(row_lo[hh * 64 + l]);
            const int I = r0 / 64 + hh;
            um[hh] = (I < p.Tr64) ? p.umax + ((size_t)bh * p.Tr64 + I) * p.Tc : nullptr;
        }
        const int n = build_list(list, p.Tc, [&](int J) {
            const int f0 = (um[0] && um[0][J] * p.scale > th[0]) ? 1 : 0;
            const int f1 = (um[1] && um[1][J] * p.scale > th[1]) ? 2 : 0;
            return f0 | f1;
        });
        if (l == 0) {
            nlist_s = n;
            ovf_s = 0;
        }
    }
    __syncthreads();

    const int srow = qh * 64 + kh * 32 + m;  // the row this lane solves (with lane l ^ 32)
    const bool svalid = (r0 + srow) < p.L;
    // per-row state: 1 = to be (re)collected and solved, 0 = solved, 2 = overflowing
    __shared__ int rstate[kBR];
    if (t < kBR) rstate[t] = (r0 + t) < p.L ? 1 : 0;
    __syncthreads();

    for (int round = 0; round < kRounds; ++round) {
        // ---- collect candidates s > tau_lo of the rows still open
        float lo_q[2];
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            const int row = qh * 64 + qb * 32 + m;
            lo_q[qb] = rstate[row] == 1 ? row_lo[row] : __builtin_inff();
        }
        ring_sweep<T, D, S>(list, nlist_s, Kh, ring, qop, R0, g, [&](int J, int, f32x16(&acc)[2][2]) {
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
                float bm = neg_inf();
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) bm = fmaxf(bm, acc[kb][qb][r]);
                if (__ballot(bm * p.scale > lo_q[qb]) == 0) continue;
                const int row = qh * 64 + qb * 32 + m;
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const float sv = acc[kb][qb][r] * p.scale;
                        if (sv > lo_q[qb]) {
                            const int slot = atomicAdd(&cnt[row], 1);
                            if (slot < cap) {
                                cval[row * CST + slot] = sv;
                                cjt[row * CST + slot] = (uint16_t)J;
                            }
                        }
                    }
            }
        });

        // ---- solve the open rows whose lists are complete; for overflowing
        // rows, the threshold of the candidates they kept is a better bound
        const int st0 = rstate[srow];
        const int nc = cnt[srow];
        const bool open = st0 == 1;
        const bool complete = open && nc <= cap;
        const int n = nc < cap ? nc : cap;
        const float* cv = cval + srow * CST;
        const double mx = row_m[srow];
        const double tau_row = solve_candidates(cv, n, mx, row_lo[srow],
                                                mx - 2.0 / sqrt((double)(nc > 0 ? nc : 1)), complete, h);
        // subset threshold (a lower bound on the row's tau) for overflowing rows
        const bool over = open && nc > cap;
        const float smax = list_max(cv, n, h);
        const double tau_sub = solve_candidates(cv, n, smax, (double)smax - 2.0,
                                                (double)smax - 2.0 / sqrt((double)(n > 0 ? n : 1)), over, h);
        if (complete) {
            const float tr = (float)tau_row;
            for (int i = h; i < n; i += 2)
                if (cv[i] > tr) {
                    const int J = cjt[srow * CST + i];
                    atomicOr(&maskw[qh][J >> 5], 1u << (J & 31));
                }
        }
        __syncthreads();  // every lane is done reading the lists
        if (h == 0) {
            if (complete) {
                row_tau[srow] = (float)tau_row;
                rstate[srow] = 0;
            } else if (over) {
                // upper bracket from this round's count of scores above tau_lo
                fb_part[srow][0][1] = (float)(mx - 2.0 / sqrt((double)nc));
                const float nl = fmaxf(row_lo[srow], (float)tau_sub);
                // no progress possible: leave the row to the sweep fallback
                if (round == kRounds - 1 || !(nl > row_lo[srow])) rstate[srow] = 2;
                row_lo[srow] = nl;
                cnt[srow] = 0;
            }
        }
        if (t == 0) ovf_s = 0;
        __syncthreads();
        if (h == 0 && rstate[srow] == 1) atomicOr(&ovf_s, 1);
        __syncthreads();
        if (!ovf_s) break;
    }
    if (t == 0) ovf_s = 0;
    __syncthreads();
    if (h == 0 && rstate[srow] == 2) {
        atomicOr(&ovf_s, 1);
        fb_part[srow][0][0] = row_lo[srow];
    }
    __syncthreads();

    // ---- fallback: Halley-bisection sweeps for rows whose list overflowed
    if (ovf_s) {
        // per-row state in LDS: lo in row_lo, hi in row_m's sibling array
        __shared__ float fb_lo[kBR], fb_hi[kBR], fb_t[kBR];
        __shared__ int fb_active[kBR];
        __shared__ int fb_any;
        if (h == 0) {
            const bool ovf = svalid && rstate[srow] == 2;
            fb_active[srow] = ovf ? 1 : 0;
            fb_lo[srow] = ovf ? fb_part[srow][0][0] : 0.f;
            fb_hi[srow] = ovf ? fb_part[srow][0][1] : 0.f;
            fb_t[srow] = ovf ? fb_part[srow][0][0] : 0.f;
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
            ring_sweep<T, D, S>(list, nlist_s, Kh, ring, qop, R0, g, [&](int, int, f32x16(&acc)[2][2]) {
#pragma unroll
                for (int qb = 0; qb < 2; ++qb) {
                    if (!aq[qb]) continue;
#pragma unroll
                    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const float s = acc[kb][qb][r] * p.scale;
                            if (s > tq[qb]) {
                                const float gg = 0.5f * (s - tq[qb]);
                                sc[qb] += 1.f;
                                sf[qb] += gg * gg;
                                sf1[qb] += gg;
                            }
                        }
                }
            });
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
            if (t == 0) fb_any = 0;
            __syncthreads();
            if (h == 0 && fb_active[srow]) {
                const float C = fb_part[srow][0][0] + fb_part[srow][1][0];
                const float F = fb_part[srow][0][1] + fb_part[srow][1][1];
                const float F1 = fb_part[srow][0][2] + fb_part[srow][1][2];
                float lo = fb_lo[srow], hi = fb_hi[srow], tc = fb_t[srow];
                if (F - 1.0f >= 0.0f) lo = tc; else hi = tc;
                if (hi - lo <= 4e-7f * fmaxf(1.0f, fabsf(tc))) {
                    fb_active[srow] = 0;
                    row_tau[srow] = 0.5f * (lo + hi);
                } else {
                    fb_t[srow] = halley_or_bisect(tc, F, F1, C, lo, hi);
                    atomicOr(&fb_any, 1);
                }
                fb_lo[srow] = lo;
                fb_hi[srow] = hi;
            }
            __syncthreads();
            if (!fb_any) break;
        }
        // rows still active after the cap take their bracket midpoint
        if (h == 0 && fb_active[srow]) row_tau[srow] = 0.5f * (fb_lo[srow] + fb_hi[srow]);
        __syncthreads();
        // mark the tiles of the overflow rows
        float tq[2];
        bool aq[2];
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            const int row = qh * 64 + qb * 32 + m;
            aq[qb] = (r0 + row) < p.L && rstate[row] == 2;
            tq[qb] = row_tau[row];
        }
        ring_sweep<T, D, S>(list, nlist_s, Kh, ring, qop, R0, g, [&](int J, int, f32x16(&acc)[2][2]) {
            bool any = false;
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
                if (!aq[qb]) continue;
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) any |= acc[kb][qb][r] * p.scale > tq[qb];
            }
            if (__ballot(any) != 0 && l == 0) atomicOr(&maskw[qh][J >> 5], 1u << (J & 31));
        });
    }

    // ---- outputs: tau and the packed mask of both 64-row blocks
    if (t < kBR) {
        const int row = r0 + t;
        if (row < p.L) p.tau[(size_t)bh * p.L + row] = row_tau[t];
    }
    for (int i = t; i < 2 * p.Wd; i += kNT) {
        const int hh = i / p.Wd, wd = i % p.Wd;
        const int I = r0 / 64 + hh;
        if (I < p.Tr64) p.mask[((size_t)bh * p.Tr64 + I) * p.Wd + wd] = maskw[hh][wd];
    }
}

// ------------------------------------------------------------ kernel 2
template <typename T, int D>
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

    const int t = threadIdx.x, w = t / kWave, qh = w & 1, kh = w >> 1;
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
        // 4A = [s - tau]_+^2 with s = scale * (Q.K)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int qb = 0; qb < 2; ++qb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float dd = fmaxf(acc[kb][qb][r] * p.scale - tq[qb], 0.0f);
                    acc[kb][qb][r] = dd * dd;
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

template <typename T, int D>
hipError_t launch_typed(const FwdParams& fp, int grid, int phase, hipStream_t stream) {
    if (phase & 1) {
        if (fp.Tc <= 128)
            hipLaunchKernelGGL((fwd_stats_kernel<T, D, 128>), dim3(grid), dim3(kNT), 0, stream, fp);
        else if (fp.Tc <= 256)
            hipLaunchKernelGGL((fwd_stats_kernel<T, D, 256>), dim3(grid), dim3(kNT), 0, stream, fp);
        else
            hipLaunchKernelGGL((fwd_stats_kernel<T, D, kMaxTc>), dim3(grid), dim3(kNT), 0, stream, fp);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (phase & 2) {
        hipLaunchKernelGGL((fwd_solve_kernel<T, D>), dim3(grid), dim3(kNT), 0, stream, fp);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (phase & 4) {
        hipLaunchKernelGGL((fwd_out_kernel<T, D>), dim3(grid), dim3(kNT), 0, stream, fp);
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

}  // namespace
}  // namespace attn

size_t attn_threshold_workspace_bytes(int B, int H, int L) {
    return attn::round256(attn::rowstat_bytes(B, H, L)) + attn::round256(attn::umax_bytes(B, H, L));
}

size_t attn_fwd_workspace_bytes(int B, int H, int L, int, int) {
    // threshold scratch, then room for the block mask when the caller does not keep it
    return attn_threshold_workspace_bytes(B, H, L) + attn::round256(attn::mask_bytes(B, H, L));
}

int attn_max_candidate_cap(int d, int dtype) {
    if (dtype == 1 && d == 64) return attn::FwdCfg<__bf16, 64>::kCap;
    return attn::FwdCfg<__bf16, 128>::kCap;
}

hipError_t launch_attn_fwd(const AttnArgs& a, int phase, hipStream_t stream) {
    using namespace attn;
    if (a.L > kMaxL) return hipErrorInvalidValue;
    FwdParams fp;
    fp.q = a.q; fp.k = a.k; fp.v = a.v; fp.o = a.o; fp.tau = a.tau;
    char* ws = reinterpret_cast<char*>(a.workspace);
    fp.rowstat = reinterpret_cast<float*>(ws);
    fp.umax = reinterpret_cast<float*>(ws + round256(rowstat_bytes(a.B, a.H, a.L)));
    fp.mask = a.block_mask ? a.block_mask
                           : reinterpret_cast<uint32_t*>(ws + attn_threshold_workspace_bytes(a.B, a.H, a.L));
    fp.BH = a.B * a.H; fp.L = a.L; fp.mode = a.mask; fp.W = a.window;
    fp.nQ = (a.L + kBR - 1) / kBR;
    fp.Tc = (a.L + kBC - 1) / kBC;
    fp.Tr64 = (a.L + 63) / 64;
    fp.Wd = (fp.Tc + 31) / 32;
    fp.scale = a.scale;
    fp.cap = a.cand_cap;
    const int grid = fp.nQ * fp.BH;
    if (a.dtype == 1) {
        if (a.d == 64) return launch_typed<__bf16, 64>(fp, grid, phase, stream);
        return launch_typed<__bf16, 128>(fp, grid, phase, stream);
    }
    if (a.d == 64) return launch_typed<float, 64>(fp, grid, phase, stream);
    return launch_typed<float, 128>(fp, grid, phase, stream);
}

}  // namespace entmax
