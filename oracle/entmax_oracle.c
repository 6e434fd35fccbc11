/*
 * entmax_oracle.c -- plain fp64 CPU oracle for 1.5-entmax attention.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the independent reference that the
 * GPU path is checked against.  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load it; the product library never
 * does, and it shares no code, header or constant with the HIP sources.
 *
 * What it computes, and where the pages define it:
 *
 *  - 1.5-entmax of a score vector s:  p_j = [(s_j - tau)/2]_+^2 with tau the
 *    unique value making sum_j p_j = 1.  ("GPT-2 with AdaSplash Attention via
 *    NeuralOps", Mathematical Formulation item 2; "DistilBERT MNLI with
 *    AdaSplash Attention via NeuralOps", Mathematical Formulation item 2;
 *    "AdaSplash-2: Faster Differentiable Sparse Attention", sec. 2.3 and the
 *    normaliser f(tau) of sec. 2.4, written there with tau' = tau/2.)
 *    Entries equal to -inf are masked out and take no part in the row.
 *
 *  - tau is found exactly, with no iteration, by the sorting method that
 *    AdaSplash-2 sec. 2.4 ("Sorting-based solvers") names for alpha = 1.5:
 *    the support is a top-k set of the sorted scores, and for a fixed support
 *    the normaliser is a quadratic in tau whose coefficients are the count,
 *    sum and sum of squares of the support (the S0, S1, S2 of AdaSplash-2
 *    appendix C.3).  The smaller root is the one below the support scores.
 *
 *  - Attention: S = scale * Q K^T over the active keys of each query row,
 *    O = A V with A the row-wise 1.5-entmax of S (AdaSplash-2 sec. 2.2).
 *    Active keys per mask mode (0-indexed positions):
 *       0 none:                 every key
 *       1 causal:               j <= i
 *       2 causal window + sink: j <= i and (j == 0 or i - j <= window)
 *    Mode 2 is the causal "splash" mask of the GPT-2 model card (item 1 of
 *    its Mathematical Formulation): key 0 always active plus the keys no more
 *    than W positions behind the query.
 *
 *  - Backward, by implicit differentiation of the normaliser (gradients live
 *    on the support only, AdaSplash-2 sec. 3.3 "Backward pass"):
 *       g_ij  = [(s_ij - tau_i)/2]_+          (so A_ij = g_ij^2)
 *       dA_ij = dO_i . V_j
 *       delta_i = sum_j g_ij dA_ij / sum_j g_ij
 *       dS_ij = g_ij (dA_ij - delta_i)
 *       dQ_i = scale sum_j dS_ij K_j,  dK_j = scale sum_i dS_ij Q_i,
 *       dV_j = sum_i A_ij dO_i.
 *
 *  - Block mask: M[I][J] = 1 iff some query of row block I has a key of
 *    column block J with A > 0 (AdaSplash-2 sec. 3.3 Phase 3, appendix C.4),
 *    packed 32 column blocks per uint32, bit (J mod 32) of word J / 32.
 *
 * General alpha in (1, 2] (AdaSplash-2 sec. 2.3, alpha-entmax; its solvers in
 * sec. 2.4), in the same score units: with e = 1/(alpha - 1),
 *       p_j = [(alpha - 1)(s_j - tau)]_+^e,   sum_j p_j = 1
 * (the pages write (alpha - 1) s_j - tau' with tau' = (alpha - 1) tau; for
 * alpha = 1.5 this is the map above).  tau lies in the bracket
 * [m - 1/(alpha-1), m - n^(1-alpha)/(alpha-1)] of AdaSplash-2 sec. 2.4
 * (p_max between 1/n and 1).  alpha = 1.5 keeps the quadratic above;
 * alpha = 2 (sparsemax) is exact by sorting: for the top-k set the
 * normaliser sum_{t<=k} (x_t - tau) = 1 is linear, tau_k = (sum_{t<=k} x_t
 * - 1)/k, and the support is the largest k with x_k > tau_k; any other alpha
 * is solved by bisection on the bracket down to fp64 resolution.  The backward
 * keeps its form with g_ij = [(alpha - 1)(s_ij - tau_i)]_+^(e - 1), the
 * derivative of p_ij in s_ij (g = (s - tau)/2 at alpha = 1.5, the support
 * indicator at alpha = 2).
 *
 * All arithmetic is fp64; inputs arrive as fp32 arrays (bf16 and fp32 values
 * are both exactly representable there).  Sums run in index order.  Exact
 * zeros of A are skipped in the products, which changes no result.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int orc_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

static int cmp_desc(const void* a, const void* b) {
    double x = *(const double*)a, y = *(const double*)b;
    return (x < y) - (x > y);
}

/*
 * Exact tau of one row.  s[0..n) with -INFINITY marking inactive entries.
 * work must hold n doubles.  Returns tau (-INFINITY for a row with no active
 * entry) and writes the support size to *k_out when k_out is not NULL.
 *
 * Sorted descending x_1 >= ... >= x_n, shifted by the max m (y = x - m, so
 * y_1 = 0).  For the top-k set the normaliser sum_t ((y_t - t)/2)^2 = 1 reads
 * k t^2 - 2 a_k t + (b_k - 4) = 0 with a_k = sum y_t and b_k = sum y_t^2.
 * Its smaller root t_k = (a_k - sqrt(a_k^2 - k (b_k - 4))) / k is the
 * threshold of that support; the true support is the largest k whose root
 * lies at or below its own k-th score (t_k <= y_k).  k = 1 always qualifies
 * (t_1 = -2), which is the lower bracket end tau >= max - 2.
 */
double orc_entmax15_tau(const double* s, int64_t n, double* work, int64_t* k_out) {
    int64_t na = 0;
    for (int64_t j = 0; j < n; ++j)
        if (s[j] != -INFINITY) work[na++] = s[j];
    if (na == 0) {
        if (k_out) *k_out = 0;
        return -INFINITY;
    }
    qsort(work, (size_t)na, sizeof(double), cmp_desc);
    const double m = work[0];
    double a = 0.0, b = 0.0, best = -2.0;
    int64_t kbest = 1;
    for (int64_t k = 1; k <= na; ++k) {
        const double y = work[k - 1] - m;
        a += y;
        b += y * y;
        const double disc = a * a - (double)k * (b - 4.0);
        if (disc < 0.0) continue;
        const double t = (a - sqrt(disc)) / (double)k;
        if (t <= y) {
            best = t;
            kbest = k;
        }
    }
    if (k_out) *k_out = kbest;
    return m + best;
}

/* p_j = [(s_j - tau)/2]_+^2 for one row; returns tau. */
double orc_entmax15(const double* s, int64_t n, double* p, int64_t* k_out) {
    double* work = (double*)malloc((size_t)(n > 0 ? n : 1) * sizeof(double));
    const double tau = orc_entmax15_tau(s, n, work, k_out);
    for (int64_t j = 0; j < n; ++j) {
        const double g = (s[j] > tau) ? 0.5 * (s[j] - tau) : 0.0;
        p[j] = g * g;
    }
    free(work);
    return tau;
}

/* [u]_+^e for the alpha-entmax map (u = (alpha - 1)(s - tau)). */
static double pos_pow(double u, double e) {
    if (!(u > 0.0)) return 0.0;
    if (e == 1.0) return u;
    if (e == 2.0) return u * u;
    return pow(u, e);
}

/* Exact sparsemax threshold (alpha = 2) of the n active entries of s: sort
 * descending, tau_k = (sum_{t<=k} x_t - 1)/k, support = largest k with
 * x_k > tau_k (k = 1 always qualifies). */
static double sparsemax_tau(const double* s, int64_t n, double* work, int64_t* k_out) {
    int64_t na = 0;
    for (int64_t j = 0; j < n; ++j)
        if (s[j] != -INFINITY) work[na++] = s[j];
    if (na == 0) {
        if (k_out) *k_out = 0;
        return -INFINITY;
    }
    qsort(work, (size_t)na, sizeof(double), cmp_desc);
    double c = 0.0, best = work[0] - 1.0;
    int64_t kbest = 1;
    for (int64_t k = 1; k <= na; ++k) {
        c += work[k - 1];
        const double t = (c - 1.0) / (double)k;
        if (work[k - 1] > t) {
            best = t;
            kbest = k;
        }
    }
    if (k_out) *k_out = kbest;
    return best;
}

/* Bisection for any alpha in (1, 2] on the bracket
 * [m - 1/(alpha-1), m - n^(1-alpha)/(alpha-1)]: f(t) = sum p_j(t) - 1 is
 * decreasing, >= 0 at the lower end and <= 0 at the upper end.  Halves until
 * the midpoint no longer moves (fp64 resolution). */
double orc_entmax_tau_bisect(const double* s, int64_t n, double alpha) {
    const double e = 1.0 / (alpha - 1.0);
    double m = -INFINITY;
    int64_t na = 0;
    for (int64_t j = 0; j < n; ++j)
        if (s[j] != -INFINITY) {
            m = s[j] > m ? s[j] : m;
            ++na;
        }
    if (na == 0) return -INFINITY;
    double lo = m - e, hi = m - pow((double)na, 1.0 - alpha) * e;
    for (int it = 0; it < 2000; ++it) {
        const double mid = 0.5 * (lo + hi);
        if (mid <= lo || mid >= hi) break;
        double f = -1.0;
        for (int64_t j = 0; j < n; ++j)
            if (s[j] != -INFINITY) f += pos_pow((alpha - 1.0) * (s[j] - mid), e);
        if (f >= 0.0) lo = mid;
        else hi = mid;
    }
    return 0.5 * (lo + hi);
}

/* tau of one row for alpha in (1, 2]; *k_out = support size. */
double orc_entmax_tau_alpha(const double* s, int64_t n, double alpha, double* work,
                            int64_t* k_out) {
    if (alpha == 1.5) return orc_entmax15_tau(s, n, work, k_out);
    double t;
    if (alpha == 2.0) {
        t = sparsemax_tau(s, n, work, k_out);
    } else {
        t = orc_entmax_tau_bisect(s, n, alpha);
        if (k_out) {
            int64_t k = 0;
            for (int64_t j = 0; j < n; ++j) k += (s[j] != -INFINITY) && (s[j] > t);
            *k_out = k;
        }
    }
    return t;
}

/*
 * Histogram threshold of AdaSplash-2 sec. 3.1 / appendix C.3 for one row, in
 * score units.  z_j = (alpha-1)(s_j - m) + 1 (the pages' (alpha-1)s - (m'-1)
 * with m' = (alpha-1) max s) is formed in fp64 from the fp32 inputs, binned
 * into B left-edge bins k = min(floor(B z), B - 1) for z >= 0; the histogram
 * objective sum_k H_k [k/B - tau]_+^e = 1 is then solved in fp64: by the
 * sorting scan over the bins (from the top) for alpha = 1.5 (a quadratic per
 * prefix) and alpha = 2 (linear), by bisection otherwise.  Proposition 3.1 of
 * the pages: tau* - h < tau_h <= tau* with h = 1/(B (alpha-1)) in score units.
 */
double orc_entmax_tau_histogram(const float* s, int64_t n, float alpha, int B) {
    double m = -INFINITY;
    for (int64_t j = 0; j < n; ++j) m = (double)s[j] > m ? (double)s[j] : m;
    if (m == -INFINITY) return -INFINITY;
    const double a1 = (double)alpha - 1.0, e = 1.0 / a1;
    double* H = (double*)calloc((size_t)B, sizeof(double));
    for (int64_t j = 0; j < n; ++j) {
        if (s[j] == -INFINITY) continue;
        const double z = a1 * ((double)s[j] - m) + 1.0;
        if (!(z >= 0.0)) continue;
        int k = (int)floor(z * (double)B);
        if (k > B - 1) k = B - 1;
        if (k < 0) k = 0;
        H[k] += 1.0;
    }
    double tz;
    if (alpha == 1.5f || alpha == 2.0f) {
        /* prefix scan over the bins from the top; the support of the binned
         * problem is the largest prefix whose root lies below its lowest edge */
        double S0 = 0.0, S1 = 0.0, S2 = 0.0;
        tz = (double)(B - 1) / B - 1.0;
        for (int k = B - 1; k >= 0; --k) {
            if (H[k] == 0.0) continue;
            const double x = (double)k / B;
            S0 += H[k];
            S1 += H[k] * x;
            S2 += H[k] * x * x;
            double t;
            if (alpha == 2.0f) {
                t = (S1 - 1.0) / S0;
            } else {
                /* sum H_k (x_k - t)^2 = 1:  S0 t^2 - 2 S1 t + S2 - 1 = 0 */
                const double disc = S1 * S1 - S0 * (S2 - 1.0);
                if (disc < 0.0) continue;
                t = (S1 - sqrt(disc)) / S0;
            }
            if (t < x) tz = t;
        }
    } else {
        double lo = (double)(B - 1) / B - 1.0, hi = (double)(B - 1) / B;
        for (int it = 0; it < 200; ++it) {
            const double mid = 0.5 * (lo + hi);
            if (mid <= lo || mid >= hi) break;
            double f = -1.0;
            for (int k = 0; k < B; ++k) {
                const double u = (double)k / B - mid;
                if (u > 0.0 && H[k] > 0.0) f += H[k] * pow(u, e);
            }
            if (f >= 0.0) lo = mid;
            else hi = mid;
        }
        tz = 0.5 * (lo + hi);
    }
    free(H);
    return m + (tz - 1.0) * e;
}

/* Weight p and derivative g = dp/ds of one score at threshold tau. */
static double weight_alpha(double x, double tau, double alpha) {
    if (alpha == 1.5) {
        const double g = (x > tau) ? 0.5 * (x - tau) : 0.0;
        return g * g;
    }
    return (x > tau) ? pos_pow((alpha - 1.0) * (x - tau), 1.0 / (alpha - 1.0)) : 0.0;
}
static double grad_alpha(double x, double tau, double alpha) {
    if (alpha == 1.5) return (x > tau) ? 0.5 * (x - tau) : 0.0;
    if (!(x > tau)) return 0.0;
    const double e1 = 1.0 / (alpha - 1.0) - 1.0;  /* 0 at alpha = 2: g = 1 on the support */
    return e1 == 0.0 ? 1.0 : pos_pow((alpha - 1.0) * (x - tau), e1);
}

/* p of one row for alpha in (1, 2]; returns tau. */
double orc_entmax_alpha(const double* s, int64_t n, double alpha, double* p, int64_t* k_out) {
    double* work = (double*)malloc((size_t)(n > 0 ? n : 1) * sizeof(double));
    const double tau = orc_entmax_tau_alpha(s, n, alpha, work, k_out);
    for (int64_t j = 0; j < n; ++j) p[j] = weight_alpha(s[j], tau, alpha);
    free(work);
    return tau;
}

/*
 * Row-wise entmax of a materialised fp32 score matrix S[rows][ld] (cols used
 * per row).  tau[rows]; P[rows][cols] (row stride cols) may be NULL.
 */
void orc_tau_rows_alpha(const float* S, int64_t rows, int64_t cols, int64_t ld,
                        double alpha, double* tau, double* P) {
#pragma omp parallel
    {
        double* row = (double*)malloc((size_t)(cols > 0 ? cols : 1) * sizeof(double));
        double* work = (double*)malloc((size_t)(cols > 0 ? cols : 1) * sizeof(double));
#pragma omp for schedule(dynamic, 16)
        for (int64_t r = 0; r < rows; ++r) {
            for (int64_t c = 0; c < cols; ++c) row[c] = (double)S[r * ld + c];
            const double t = orc_entmax_tau_alpha(row, cols, alpha, work, NULL);
            tau[r] = t;
            if (P) {
                for (int64_t c = 0; c < cols; ++c) P[r * cols + c] = weight_alpha(row[c], t, alpha);
            }
        }
        free(row);
        free(work);
    }
}

void orc_tau_rows(const float* S, int64_t rows, int64_t cols, int64_t ld, double* tau,
                  double* P) {
    orc_tau_rows_alpha(S, rows, cols, ld, 1.5, tau, P);
}

/* Active-key predicate of the three mask modes (0-indexed positions). */
int orc_key_active(int mask, int64_t window, int64_t i, int64_t j) {
    if (mask == 0) return 1;
    if (j > i) return 0;
    if (mask == 1) return 1;
    return (j == 0) || (i - j <= window);
}

/* Scores of query row i of one head: s[j] = scale * Q_i . K_j, -inf if masked. */
static void head_row_scores(const float* Q, const float* K, int64_t L, int64_t d,
                            double scale, int mask, int64_t window, int64_t i,
                            double* s) {
    const float* q = Q + i * d;
    for (int64_t j = 0; j < L; ++j) {
        if (!orc_key_active(mask, window, i, j)) {
            s[j] = -INFINITY;
            continue;
        }
        const float* k = K + j * d;
        double acc = 0.0;
        for (int64_t c = 0; c < d; ++c) acc += (double)q[c] * (double)k[c];
        s[j] = scale * acc;
    }
}

/*
 * Attention forward for a list of query rows.  Q, K, V are [BH][L][d].
 * rows[r] indexes the flattened [BH*L] query rows; rows == NULL means all
 * BH*L rows in order (nrows must then equal BH*L).  Outputs per listed row:
 * O[r][d], tau[r], and (optional) support size nsup[r] and the sum of the
 * derivatives g over the row, gsum[r] = sum_j g_ij (sum_j [(s_j - tau)/2]_+
 * at alpha = 1.5).
 */
void orc_attn_fwd_alpha(const float* Q, const float* K, const float* V,
                        int64_t BH, int64_t L, int64_t d, double scale, int mask,
                        int64_t window, double alpha, const int64_t* rows,
                        int64_t nrows, double* O, double* tau, int64_t* nsup,
                        double* gsum) {
    (void)BH;
#pragma omp parallel
    {
        double* s = (double*)malloc((size_t)L * sizeof(double));
        double* work = (double*)malloc((size_t)L * sizeof(double));
#pragma omp for schedule(dynamic, 4)
        for (int64_t r = 0; r < nrows; ++r) {
            const int64_t flat = rows ? rows[r] : r;
            const int64_t bh = flat / L, i = flat % L;
            const float* Qh = Q + bh * L * d;
            const float* Kh = K + bh * L * d;
            const float* Vh = V + bh * L * d;
            head_row_scores(Qh, Kh, L, d, scale, mask, window, i, s);
            int64_t k = 0;
            const double t = orc_entmax_tau_alpha(s, L, alpha, work, &k);
            tau[r] = t;
            if (nsup) nsup[r] = k;
            double* o = O + r * d;
            for (int64_t c = 0; c < d; ++c) o[c] = 0.0;
            double gs = 0.0;
            for (int64_t j = 0; j < L; ++j) {
                if (!(s[j] > t)) continue; /* A_ij = 0 exactly */
                const double a = weight_alpha(s[j], t, alpha);
                gs += grad_alpha(s[j], t, alpha);
                const float* v = Vh + j * d;
                for (int64_t c = 0; c < d; ++c) o[c] += a * (double)v[c];
            }
            if (gsum) gsum[r] = gs;
        }
        free(s);
        free(work);
    }
}

void orc_attn_fwd(const float* Q, const float* K, const float* V, int64_t BH, int64_t L,
                  int64_t d, double scale, int mask, int64_t window, const int64_t* rows,
                  int64_t nrows, double* O, double* tau, int64_t* nsup, double* gsum) {
    orc_attn_fwd_alpha(Q, K, V, BH, L, d, scale, mask, window, 1.5, rows, nrows, O, tau, nsup,
                       gsum);
}

/*
 * Block masks of one head at tile br x bc.  Three masks, each
 * [ceil(L/br)][ceil(ceil(L/bc)/32)] words:
 *   m_exact: tile has an entry with s > tau            (the definition)
 *   m_lo:    tile has an entry with s - tau >  tol     (must be set)
 *   m_hi:    tile has an entry with s - tau > -tol     (may be set)
 * tau_out[L] receives the row thresholds when not NULL.
 */
void orc_block_mask_head_alpha(const float* Q, const float* K, int64_t L, int64_t d,
                               double scale, int mask, int64_t window, double alpha,
                               int64_t br, int64_t bc, double tol, uint32_t* m_exact,
                               uint32_t* m_lo, uint32_t* m_hi, double* tau_out) {
    const int64_t Tr = (L + br - 1) / br, Tc = (L + bc - 1) / bc;
    const int64_t Wd = (Tc + 31) / 32;
    memset(m_exact, 0, (size_t)(Tr * Wd) * sizeof(uint32_t));
    memset(m_lo, 0, (size_t)(Tr * Wd) * sizeof(uint32_t));
    memset(m_hi, 0, (size_t)(Tr * Wd) * sizeof(uint32_t));
    /* one row block per iteration: no two threads write the same words */
#pragma omp parallel
    {
        double* s = (double*)malloc((size_t)L * sizeof(double));
        double* work = (double*)malloc((size_t)L * sizeof(double));
#pragma omp for schedule(dynamic, 1)
        for (int64_t I = 0; I < Tr; ++I) {
            for (int64_t i = I * br; i < L && i < (I + 1) * br; ++i) {
                head_row_scores(Q, K, L, d, scale, mask, window, i, s);
                const double t = orc_entmax_tau_alpha(s, L, alpha, work, NULL);
                if (tau_out) tau_out[i] = t;
                for (int64_t j = 0; j < L; ++j) {
                    if (s[j] == -INFINITY) continue;
                    const int64_t J = j / bc;
                    const uint32_t bit = 1u << (J % 32);
                    if (s[j] > t) m_exact[I * Wd + J / 32] |= bit;
                    if (s[j] - t > tol) m_lo[I * Wd + J / 32] |= bit;
                    if (s[j] - t > -tol) m_hi[I * Wd + J / 32] |= bit;
                }
            }
        }
        free(s);
        free(work);
    }
}

void orc_block_mask_head(const float* Q, const float* K, int64_t L, int64_t d, double scale,
                         int mask, int64_t window, int64_t br, int64_t bc, double tol,
                         uint32_t* m_exact, uint32_t* m_lo, uint32_t* m_hi, double* tau_out) {
    orc_block_mask_head_alpha(Q, K, L, d, scale, mask, window, 1.5, br, bc, tol, m_exact, m_lo,
                              m_hi, tau_out);
}

/*
 * Full backward of one head.  Q, K, V, dO are [L][d]; outputs dQ, dK, dV are
 * [L][d]; tau[L], delta[L] optional.  Row pass (parallel over queries): tau,
 * the support, delta, dQ_i, and the support's (j, A_ij, dS_ij).  Column pass
 * (serial in query order per key): dK_j and dV_j from those entries.
 */
void orc_attn_bwd_head_alpha(const float* Q, const float* K, const float* V,
                             const float* dO, int64_t L, int64_t d, double scale,
                             int mask, int64_t window, double alpha, double* dQ,
                             double* dK, double* dV, double* tau_out, double* delta_out) {
    int64_t* sup_off = (int64_t*)calloc((size_t)L + 1, sizeof(int64_t));
    int64_t** sup_j = (int64_t**)calloc((size_t)L, sizeof(int64_t*));
    double** sup_a = (double**)calloc((size_t)L, sizeof(double*));
    double** sup_ds = (double**)calloc((size_t)L, sizeof(double*));
#pragma omp parallel
    {
        double* s = (double*)malloc((size_t)L * sizeof(double));
        double* work = (double*)malloc((size_t)L * sizeof(double));
#pragma omp for schedule(dynamic, 4)
        for (int64_t i = 0; i < L; ++i) {
            head_row_scores(Q, K, L, d, scale, mask, window, i, s);
            int64_t k = 0;
            const double t = orc_entmax_tau_alpha(s, L, alpha, work, &k);
            if (tau_out) tau_out[i] = t;
            int64_t cnt = 0;
            for (int64_t j = 0; j < L; ++j) cnt += (s[j] > t);
            sup_off[i + 1] = cnt;
            int64_t* jj = (int64_t*)malloc((size_t)(cnt > 0 ? cnt : 1) * sizeof(int64_t));
            double* aa = (double*)malloc((size_t)(cnt > 0 ? cnt : 1) * sizeof(double));
            double* dd = (double*)malloc((size_t)(cnt > 0 ? cnt : 1) * sizeof(double));
            double* gg = (double*)malloc((size_t)(cnt > 0 ? cnt : 1) * sizeof(double));
            double* da = (double*)malloc((size_t)(cnt > 0 ? cnt : 1) * sizeof(double));
            const float* go = dO + i * d;
            double num = 0.0, den = 0.0;
            int64_t c = 0;
            for (int64_t j = 0; j < L; ++j) {
                if (!(s[j] > t)) continue;
                const double g = grad_alpha(s[j], t, alpha);
                const float* v = V + j * d;
                double dot = 0.0;
                for (int64_t e = 0; e < d; ++e) dot += (double)go[e] * (double)v[e];
                jj[c] = j;
                gg[c] = g;
                aa[c] = weight_alpha(s[j], t, alpha);
                da[c] = dot;
                num += g * dot;
                den += g;
                ++c;
            }
            const double delta = (den > 0.0) ? num / den : 0.0;
            if (delta_out) delta_out[i] = delta;
            double* dq = dQ + i * d;
            for (int64_t e = 0; e < d; ++e) dq[e] = 0.0;
            for (int64_t q = 0; q < cnt; ++q) {
                const double ds = gg[q] * (da[q] - delta);
                dd[q] = ds;
                const float* kk = K + jj[q] * d;
                for (int64_t e = 0; e < d; ++e) dq[e] += scale * ds * (double)kk[e];
            }
            sup_j[i] = jj;
            sup_a[i] = aa;
            sup_ds[i] = dd;
            free(gg);
            free(da);
        }
        free(s);
        free(work);
    }
    memset(dK, 0, (size_t)(L * d) * sizeof(double));
    memset(dV, 0, (size_t)(L * d) * sizeof(double));
    for (int64_t i = 0; i < L; ++i) {
        const float* qi = Q + i * d;
        const float* go = dO + i * d;
        for (int64_t q = 0; q < sup_off[i + 1]; ++q) {
            const int64_t j = sup_j[i][q];
            const double a = sup_a[i][q], ds = sup_ds[i][q];
            double* dk = dK + j * d;
            double* dv = dV + j * d;
            for (int64_t e = 0; e < d; ++e) {
                dk[e] += scale * ds * (double)qi[e];
                dv[e] += a * (double)go[e];
            }
        }
        free(sup_j[i]);
        free(sup_a[i]);
        free(sup_ds[i]);
    }
    free(sup_off);
    free(sup_j);
    free(sup_a);
    free(sup_ds);
}

void orc_attn_bwd_head(const float* Q, const float* K, const float* V, const float* dO,
                       int64_t L, int64_t d, double scale, int mask, int64_t window,
                       double* dQ, double* dK, double* dV, double* tau_out,
                       double* delta_out) {
    orc_attn_bwd_head_alpha(Q, K, V, dO, L, d, scale, mask, window, 1.5, dQ, dK, dV, tau_out,
                            delta_out);
}

/*
 * dQ and delta for a list of query rows of a [BH][L][d] batch (no dK/dV):
 * cheap enough to sample at any size.  dQ[r][d], delta[r], tau[r].
 */
void orc_attn_bwd_rows_alpha(const float* Q, const float* K, const float* V,
                             const float* dO, int64_t BH, int64_t L, int64_t d,
                             double scale, int mask, int64_t window, double alpha,
                             const int64_t* rows, int64_t nrows, double* dQ,
                             double* delta_out, double* tau_out) {
    (void)BH;
#pragma omp parallel
    {
        double* s = (double*)malloc((size_t)L * sizeof(double));
        double* work = (double*)malloc((size_t)L * sizeof(double));
        double* da = (double*)malloc((size_t)L * sizeof(double));
#pragma omp for schedule(dynamic, 4)
        for (int64_t r = 0; r < nrows; ++r) {
            const int64_t flat = rows[r];
            const int64_t bh = flat / L, i = flat % L;
            const float* Qh = Q + bh * L * d;
            const float* Kh = K + bh * L * d;
            const float* Vh = V + bh * L * d;
            const float* go = dO + flat * d;
            head_row_scores(Qh, Kh, L, d, scale, mask, window, i, s);
            const double t = orc_entmax_tau_alpha(s, L, alpha, work, NULL);
            if (tau_out) tau_out[r] = t;
            double num = 0.0, den = 0.0;
            for (int64_t j = 0; j < L; ++j) {
                if (!(s[j] > t)) continue;
                const double g = grad_alpha(s[j], t, alpha);
                const float* v = Vh + j * d;
                double dot = 0.0;
                for (int64_t e = 0; e < d; ++e) dot += (double)go[e] * (double)v[e];
                da[j] = dot;
                num += g * dot;
                den += g;
            }
            const double delta = (den > 0.0) ? num / den : 0.0;
            if (delta_out) delta_out[r] = delta;
            double* dq = dQ + r * d;
            for (int64_t e = 0; e < d; ++e) dq[e] = 0.0;
            for (int64_t j = 0; j < L; ++j) {
                if (!(s[j] > t)) continue;
                const double g = grad_alpha(s[j], t, alpha);
                const double ds = g * (da[j] - delta);
                const float* kk = Kh + j * d;
                for (int64_t e = 0; e < d; ++e) dq[e] += scale * ds * (double)kk[e];
            }
        }
        free(s);
        free(work);
        free(da);
    }
}

void orc_attn_bwd_rows(const float* Q, const float* K, const float* V, const float* dO,
                       int64_t BH, int64_t L, int64_t d, double scale, int mask,
                       int64_t window, const int64_t* rows, int64_t nrows, double* dQ,
                       double* delta_out, double* tau_out) {
    orc_attn_bwd_rows_alpha(Q, K, V, dO, BH, L, d, scale, mask, window, 1.5, rows, nrows, dQ,
                            delta_out, tau_out);
}
