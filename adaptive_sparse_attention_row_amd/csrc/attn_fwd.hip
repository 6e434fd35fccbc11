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

namespace entmax {
namespace attn {
namespace {

constexpr int kTop = 8;        // tile maxima kept per row for tau_lo
constexpr int kMaxIter = 40;   // solver iterations
constexpr int kFbMaxIter = 60; // fallback sweeps

struct FwdParams {
    const void* q;
    const void* k;
    const void* v;
    float* o;
    float* tau;
    uint32_t* mask;  // [BH][Tr64][Wd]
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

// ------------------------------------------------------------ kernel 1
template <typename T, int D>
__global__ __launch_bounds__(kNT, 1) void fwd_tau_kernel(FwdParams p) {
    using O = Ops<T, D>;
    constexpr int CAP = FwdCfg<T, D>::kCap;
    constexpr int NBUF = FwdCfg<T, D>::kNBuf;

    __shared__ __attribute__((aligned(16))) T kbuf[NBUF * 2 * O::kKTile];
    __shared__ __attribute__((aligned(16))) float cval[kBR * CAP];
    __shared__ uint16_t cjt[kBR * CAP];
    __shared__ float umax[2][kMaxTc];
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

    // ---- structural tile list; init tables
    for (int i = t; i < 2 * kMaxTc; i += kNT) (&umax[0][0])[i] = neg_inf();
    for (int i = t; i < 2 * (kMaxTc / 32); i += kNT) (&maskw[0][0])[i] = 0u;
    if (w == 0) {
        const int n = build_list(list, p.Tc, [&](int J) {
            return (tile_class(J, r0, g) != kSkip ? 1 : 0) | (tile_class(J, r0 + 64, g) != kSkip ? 2 : 0);
        });
        if (l == 0) nlist_s = n;
    }
    __syncthreads();

    // ---- sweep 1: row max, top tile maxima, per-(half, tile) max
    float rmax[2] = {neg_inf(), neg_inf()};
    float top[2][kTop];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int i = 0; i < kTop; ++i) top[qb][i] = neg_inf();

    sweep<T, D, NBUF, false>(list, nlist_s, Kh, nullptr, kbuf, nullptr, qop, R0, g,
                             [&](int J, int, f32x16(&acc)[2][2], const T*) {
        float wm = neg_inf();
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            float tm = neg_inf();
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) tm = fmaxf(tm, acc[kb][qb][r]);
            tm = fmaxf(tm, __shfl_xor(tm, 32, kWave));
            rmax[qb] = fmaxf(rmax[qb], tm);
            float x = tm;
#pragma unroll
            for (int i = 0; i < kTop; ++i) {
                const float hi = fmaxf(top[qb][i], x);
                x = fminf(top[qb][i], x);
                top[qb][i] = hi;
            }
            wm = fmaxf(wm, tm);
        }
#pragma unroll
        for (int o = 16; o >= 1; o >>= 1) wm = fmaxf(wm, __shfl_xor(wm, o, kWave));
        if (l == 0) umax[qh][J] = wm;
    });

    // ---- merge the two key-parity halves of each row; tau_lo
    float* st = cval;  // [kh][row][1 + kTop] (candidate space is free here)
    constexpr int kSt = 1 + kTop;
    if (h == 0) {
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            float* e = st + (kh * kBR + qh * 64 + qb * 32 + m) * kSt;
            e[0] = rmax[qb];
#pragma unroll
            for (int i = 0; i < kTop; ++i) e[1 + i] = top[qb][i];
        }
    }
    __syncthreads();
    const int srow = qh * 64 + kh * 32 + m;  // the row this lane solves
    const bool svalid = (r0 + srow) < p.L;
    if (h == 0) {
        const float* a = st + srow * kSt;
        const float* b = st + (kBR + srow) * kSt;
        float merged[2 * kTop];
        int ia = 0, ib = 0;
#pragma unroll
        for (int i = 0; i < 2 * kTop; ++i) {
            const float va = (ia < kTop) ? a[1 + ia] : neg_inf();
            const float vb = (ib < kTop) ? b[1 + ib] : neg_inf();
            const bool ta = va >= vb;
            merged[i] = (ta ? va : vb) * p.scale;
            ia += ta ? 1 : 0;
            ib += ta ? 0 : 1;
        }
        const float mx = fmaxf(a[0], b[0]) * p.scale;
        float lo = __builtin_inff();
        if (svalid) lo = tau_of_sorted(merged);
        row_m[srow] = svalid ? mx : neg_inf();
        row_lo[srow] = lo;
        cnt[srow] = 0;
    }
    __syncthreads();

    // ---- sweep-2 tile list: tiles whose best score beats some row's tau_lo
    if (w == 0) {
        float th[2];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) th[hh] = wave_min(row_lo[hh * 64 + l]);
        const int n = build_list(list, p.Tc, [&](int J) {
            return (umax[0][J] * p.scale > th[0] ? 1 : 0) | (umax[1][J] * p.scale > th[1] ? 2 : 0);
        });
        if (l == 0) {
            nlist_s = n;
            ovf_s = 0;
        }
    }
    __syncthreads();

    // ---- sweep 2: collect candidates s > tau_lo
    float lo_q[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) lo_q[qb] = row_lo[qh * 64 + qb * 32 + m];
    sweep<T, D, NBUF, false>(list, nlist_s, Kh, nullptr, kbuf, nullptr, qop, R0, g,
                             [&](int J, int, f32x16(&acc)[2][2], const T*) {
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
                    const float s = acc[kb][qb][r] * p.scale;
                    if (s > lo_q[qb]) {
                        const int slot = atomicAdd(&cnt[row], 1);
                        if (slot < cap) {
                            cval[row * CAP + slot] = s;
                            cjt[row * CAP + slot] = (uint16_t)J;
                        }
                    }
                }
        }
    });

    // ---- exact threshold per row from its candidates (two lanes per row)
    {
        const int nc = cnt[srow];
        const bool ovf = svalid && nc > cap;
        const int n = nc < cap ? nc : cap;
        const float mx = row_m[srow];
        bool done = !svalid || ovf;
        float lo = row_lo[srow];
        float hi = mx - 2.0f / sqrtf((float)(nc > 0 ? nc : 1));
        float tcur = lo, result = lo;
        const float* cv = cval + srow * CAP;
        for (int it = 0; it < kMaxIter; ++it) {
            if (__ballot(!done) == 0) break;
            double C = 0, S1 = 0, S2 = 0, F = 0, F1 = 0;
            float mn = __builtin_inff();
            if (!done) {
                for (int i = h; i < n; i += 2) {
                    const float x = cv[i];
                    if (x > tcur) {
                        const double y = (double)x - (double)mx;
                        const double gg = 0.5 * ((double)x - (double)tcur);
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
            if (!done) {
                const double f = F - 1.0;
                if (f >= 0.0) {
                    const double disc = fmax(S1 * S1 - C * (S2 - 4.0), 0.0);
                    const double ts = (double)mx + (S1 - sqrt(disc)) / C;
                    if (ts < (double)mn) {
                        result = fmaxf((float)ts, tcur);
                        done = true;
                    } else {
                        lo = tcur;
                    }
                } else {
                    hi = tcur;
                }
                if (!done) {
                    if (hi - lo <= 1e-7f * fmaxf(1.0f, fabsf(tcur))) {
                        result = 0.5f * (lo + hi);
                        done = true;
                    } else {
                        const double fp = -F1, fpp = 0.5 * C;
                        const double den = 2.0 * fp * fp - f * fpp;
                        double tn = (double)tcur - 2.0 * f * fp / den;
                        if (!(den > 0.0) || !(tn > lo && tn < hi)) tn = 0.5 * ((double)lo + (double)hi);
                        tcur = (float)tn;
                        if (!(tcur > lo && tcur < hi)) tcur = 0.5f * (lo + hi);
                    }
                }
            }
        }
        if (svalid && !ovf && !done) result = 0.5f * (lo + hi);
        if (h == 0) {
            row_tau[srow] = (svalid && !ovf) ? result : __builtin_inff();
            if (ovf) atomicOr(&ovf_s, 1);
        }
        // mask bits from candidates above tau
        const float tr = (svalid && !ovf) ? result : __builtin_inff();
        for (int i = h; i < n; i += 2)
            if (cv[i] > tr) {
                const int J = cjt[srow * CAP + i];
                atomicOr(&maskw[qh][J >> 5], 1u << (J & 31));
            }
        // overflow rows: carry their bracket to the fallback
        if (h == 0 && ovf) {
            fb_part[srow][0][0] = row_lo[srow];
            fb_part[srow][0][1] = mx - 2.0f / sqrtf((float)nc);
        }
    }
    __syncthreads();

    // ---- fallback: Halley-bisection sweeps for rows whose list overflowed
    if (ovf_s) {
        // per-row state in LDS: lo in row_lo, hi in row_m's sibling array
        __shared__ float fb_lo[kBR], fb_hi[kBR], fb_t[kBR];
        __shared__ int fb_active[kBR];
        __shared__ int fb_any;
        if (h == 0) {
            const bool ovf = svalid && cnt[srow] > cap;
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
            sweep<T, D, NBUF, false>(list, nlist_s, Kh, nullptr, kbuf, nullptr, qop, R0, g,
                                     [&](int, int, f32x16(&acc)[2][2], const T*) {
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
                if (hi - lo <= 1e-7f * fmaxf(1.0f, fabsf(tc))) {
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
            aq[qb] = (r0 + row) < p.L && cnt[row] > cap;
            tq[qb] = row_tau[row];
        }
        sweep<T, D, NBUF, false>(list, nlist_s, Kh, nullptr, kbuf, nullptr, qop, R0, g,
                                 [&](int J, int, f32x16(&acc)[2][2], const T*) {
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
        hipLaunchKernelGGL((fwd_tau_kernel<T, D>), dim3(grid), dim3(kNT), 0, stream, fp);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (phase & 2) {
        hipLaunchKernelGGL((fwd_out_kernel<T, D>), dim3(grid), dim3(kNT), 0, stream, fp);
        return hipGetLastError();
    }
    return hipSuccess;
}

size_t mask_bytes(int B, int H, int L) {
    const size_t tr = (L + 63) / 64, tc = (L + 63) / 64, wd = (tc + 31) / 32;
    return (size_t)B * H * tr * wd * sizeof(uint32_t);
}

}  // namespace
}  // namespace attn

size_t attn_fwd_workspace_bytes(int B, int H, int L, int, int) {
    // room for the block mask when the caller does not want it
    return (attn::mask_bytes(B, H, L) + 255) & ~(size_t)255;
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
    fp.mask = a.block_mask ? a.block_mask : reinterpret_cast<uint32_t*>(a.workspace);
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
