/*
 * entmax.h -- C ABI of libentmax.so: 1.5-entmax attention with a per-row
 * threshold on AMD Instinct MI355X (gfx950).
 *
 * The operation (score units throughout):
 *   S_ij  = scale * Q_i . K_j                  for active keys j of row i
 *   tau_i : sum_j [(S_ij - tau_i)/2]_+^2 = 1    (unique; the row normaliser)
 *   A_ij  = [(S_ij - tau_i)/2]_+^2              (exact zeros where S_ij <= tau_i)
 *   O_i   = sum_j A_ij V_j
 * Sources: "GPT-2 with AdaSplash Attention via NeuralOps", Mathematical
 * Formulation items 1-2 (threshold equation, masking); "AdaSplash-2: Faster
 * Differentiable Sparse Attention", sec. 2.2 (S = QK^T/sqrt(d), O = pi(S)V),
 * sec. 2.3-2.4 (alpha-entmax and its normaliser; written there as
 * [(alpha-1)s - tau']_+^(1/(alpha-1)), which is this map with tau = 2 tau'
 * for alpha = 1.5), sec. 3.3 (block mask, output over non-null blocks,
 * backward on the support).
 *
 * Conventions shared by every entry point:
 *  - Every pointer argument is DEVICE memory owned by the caller; the library
 *    never allocates, frees, or reads device data on the host.
 *  - Calls are asynchronous on `stream` (a hipStream_t passed as void*; NULL
 *    is the null stream).  Nothing synchronises.
 *  - Arguments are validated before any launch; on any error nothing is
 *    launched and no output is touched.  A failed launch returns
 *    ENTMAX_ERR_HIP (the HIP error is consumed).
 *  - alpha must lie in (1, 2]; other values (and NaN) return
 *    ENTMAX_ERR_ALPHA.  alpha = 1.5 is the map above and keeps its exact
 *    closed-form solves; any other alpha uses the alpha-entmax map of
 *    AdaSplash-2 sec. 2.3 in the same score units,
 *      A_ij = [(alpha-1)(S_ij - tau_i)]_+^(1/(alpha-1)),
 *    with tau_i from Newton steps from below (bisection-guarded); alpha = 2
 *    is sparsemax.
 *  - Outputs are overwritten, never accumulated into.
 *  - The library keeps no mutable host state: every choice a call makes comes
 *    from its own arguments (the _ex variants take an options struct).
 *    Concurrent calls on different streams are safe when their outputs and
 *    workspaces are disjoint.  The one exception is entmax_attn_decode_noalloc,
 *    whose calls on one device share a static scratch (see there).
 */
#ifndef ENTMAX_H
#define ENTMAX_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    ENTMAX_OK = 0,
    ENTMAX_ERR_NULL = 1,      /* a required pointer is NULL */
    ENTMAX_ERR_SHAPE = 2,     /* unsupported or inconsistent size */
    ENTMAX_ERR_ALPHA = 3,     /* alpha outside (1, 2] */
    ENTMAX_ERR_DTYPE = 4,     /* unknown dtype code */
    ENTMAX_ERR_MASK = 5,      /* unknown mask mode, or window < 0 in mode 2 */
    ENTMAX_ERR_WORKSPACE = 6, /* workspace missing or too small */
    ENTMAX_ERR_ALIGN = 7,     /* a pointer is not 16-byte aligned */
    ENTMAX_ERR_HIP = 8,       /* a HIP launch failed */
    ENTMAX_ERR_ARG = 9,       /* other invalid argument (scale, option) */
    ENTMAX_ERR_SCRATCH = 10   /* input larger than the static scratch of the
                                 allocation-free entry point */
};

/* Mask modes (0-indexed positions i = query, j = key).
 *  ENTMAX_MASK_NONE:  every key.
 *  ENTMAX_MASK_CAUSAL: j <= i.
 *  ENTMAX_MASK_CAUSAL_WINDOW_SINK: j <= i and (j == 0 or i - j <= window):
 *    the sink token 0 plus the keys at most `window` positions behind the
 *    query ("GPT-2 with AdaSplash Attention via NeuralOps", Mathematical
 *    Formulation item 1, active set {0} U [max(1, i - W), i]). */
enum { ENTMAX_MASK_NONE = 0, ENTMAX_MASK_CAUSAL = 1, ENTMAX_MASK_CAUSAL_WINDOW_SINK = 2 };

/* Element type of Q, K, V and dO.  O, tau and all gradients are fp32. */
enum { ENTMAX_F32 = 0, ENTMAX_BF16 = 1 };

/* Human-readable name of a status code (static string, never NULL). */
const char* entmax_status_str(int status);

/* ABI version, (major << 16) | minor. */
int entmax_version(void);

/*
 * Granularity of the block mask written by entmax_attn_fwd: row blocks of
 * *block_rows queries by column blocks of *block_cols keys (the B_r x B_c
 * tiles of AdaSplash-2 appendix C.1).  Returns ENTMAX_ERR_SHAPE for an
 * unsupported d, ENTMAX_ERR_DTYPE for an unknown dtype, ENTMAX_ERR_NULL for
 * NULL outputs.
 */
int entmax_tile_shape(int d, int dtype, int* block_rows, int* block_cols);

/*
 * Row-wise alpha-entmax (1.5-entmax for alpha = 1.5) of a materialised
 * fp32 score matrix.
 *   S    [rows][ld] fp32, row r's scores are S[r*ld + 0 .. cols-1]; -inf
 *        entries are inactive (p = 0, not counted in the row).
 *   P    [rows][ld] fp32 output (same layout as S) or NULL for tau only.
 *        P may not overlap S.
 *   tau  [rows] fp32 output, score units; -inf for a row with no finite
 *        entry (its P row is all zero).
 * Requires rows >= 0, 1 <= cols <= ld.  rows == 0 is a no-op (any pointer
 * may then be NULL); otherwise S and tau must be non-NULL.
 * The threshold solve (alpha = 1.5) is the hybrid Halley-bisection of
 * "AdaSplash: Adaptive Sparse Flash Attention" (summary, Approach) on the
 * bracket [max - 2, max - 2/sqrt(n)] of AdaSplash-2 sec. 2.4 (scaled to score
 * units; [max - 1/(alpha-1), max - n^(1-alpha)/(alpha-1)] for other alpha,
 * solved by bisection-guarded Newton steps from below),
 * restricted to the scores above a lower bound on tau taken from a subset of
 * the row (at least max - 2, less a relative 1e-5 rounding margin), with an
 * exact finish once the support is known.  NaN inputs give unspecified
 * results.
 */
int entmax_tau_rows(const float* S, float* P, float* tau, int64_t rows, int64_t cols,
                    int64_t ld, float alpha, void* stream);

/*
 * Workspace bytes entmax_attn_fwd needs: per-row statistics of the score
 * sweep (8 bytes per query row), the largest score of every (64-row block,
 * 64-key tile) (4 bytes each), per query row (L rounded up to 128) a list of
 * up to 128 candidate scores with their key indices (1024 bytes per row),
 * 4 bytes per 128-row block, plus room for the block mask (used only when
 * block_mask == NULL).  entmax_attn_threshold needs the same minus the
 * mask part: entmax_attn_threshold_workspace.  Both return 0 for invalid
 * arguments; the calls report those.
 */
size_t entmax_attn_threshold_workspace(int B, int H, int L, int d, int dtype, int mask,
                                       int window);
size_t entmax_attn_fwd_workspace(int B, int H, int L, int d, int dtype, int mask,
                                 int window);

/*
 * alpha-entmax attention forward (AdaSplash-2 sec. 3.3, phases: score sweep,
 * threshold, block mask, output over non-null blocks only).
 *   Q, K, V    [B][H][L][d] of `dtype`, contiguous, 16-byte aligned.
 *   O          [B][H][L][d] fp32 output.
 *   tau        [B][H][L] fp32 output, score units.
 *   block_mask optional output (NULL to skip): uint32
 *              [B][H][ceil(L/br)][ceil(ceil(L/bc)/32)] with (br, bc) from
 *              entmax_tile_shape; bit (J % 32) of word J/32 of row block I is
 *              set iff some query of block I has a key of block J with
 *              A > 0 (AdaSplash-2 appendix C.4 packing).
 *   scale > 0 multiplies Q.K (e.g. 1/sqrt(d)).
 *   d in {64, 128}; B, H >= 1; 1 <= L <= 65536 (per-row tile tables are
 *   kept on chip); otherwise ENTMAX_ERR_SHAPE.
 *   workspace  16-byte aligned, at least entmax_attn_fwd_workspace(...) bytes
 *              (entmax_attn_threshold_workspace(...) suffices when block_mask
 *              is not NULL).  Contents on entry are ignored.
 */
int entmax_attn_fwd(const void* Q, const void* K, const void* V, float* O, float* tau,
                    uint32_t* block_mask, int B, int H, int L, int d, float scale,
                    float alpha, int dtype, int mask, int window, void* workspace,
                    size_t workspace_bytes, void* stream);

/*
 * The two halves of entmax_attn_fwd, callable on their own (same argument
 * rules; entmax_attn_fwd is exactly threshold followed by output).
 *  entmax_attn_threshold: phases 1-3 of AdaSplash-2 sec. 3.3 -- writes tau
 *    [B][H][L] and the packed block mask (required here, same layout as
 *    above).  Needs entmax_attn_threshold_workspace(...) bytes of workspace.
 *  entmax_attn_output: phase 4 -- given that tau and block mask, writes
 *    O [B][H][L][d] fp32 from the non-null tiles only.
 */
int entmax_attn_threshold(const void* Q, const void* K, float* tau, uint32_t* block_mask,
                          int B, int H, int L, int d, float scale, float alpha, int dtype,
                          int mask, int window, void* workspace, size_t workspace_bytes,
                          void* stream);
/*
 * Phase 1 alone (AdaSplash-2 sec. 3.3 "Phase 1 (maximum)", extended): one
 * dense MFMA sweep of S = scale Q K^T over the keys the mask allows.  Writes
 * into the workspace, for each query row, its maximum score and a lower
 * bound on tau (the exact threshold of its largest tile maxima; adding scores
 * to a row only raises its threshold), as float2 [B][H][L] at offset 0, and
 * the largest raw dot product of every (64-row block, 64-key tile) as float
 * [B][H][ceil(L/64)][ceil(L/64)] at the next 256-byte boundary.
 * entmax_attn_threshold runs this and then the solve.  Workspace as for
 * entmax_attn_threshold.
 */
int entmax_attn_score_stats(const void* Q, const void* K, int B, int H, int L, int d, float scale,
                            float alpha, int dtype, int mask, int window, void* workspace,
                            size_t workspace_bytes, void* stream);
int entmax_attn_output(const void* Q, const void* K, const void* V, const float* tau,
                       const uint32_t* block_mask, float* O, int B, int H, int L, int d,
                       float scale, float alpha, int dtype, int mask, int window,
                       void* stream);

/*
 * Workspace bytes entmax_attn_bwd needs: delta per query row (4 B each,
 * rounded up to 256 B) and 4 KiB for the largest magnitudes of Q, K, V and
 * dO, from which the bf16 path scales its fp16 weight products.
 */
size_t entmax_attn_bwd_workspace(int B, int H, int L, int d, int dtype, int mask,
                                 int window);

/*
 * alpha-entmax attention backward, restricted to the support (AdaSplash-2
 * sec. 3.3 "Backward pass" and appendix C.6): with g = [(S - tau)/2]_+
 * at alpha = 1.5 (in general g = dA/dS = [(alpha-1)(S - tau)]_+^(1/(alpha-1)
 * - 1), the support indicator at alpha = 2),
 *   dA_ij = dO_i . V_j,  delta_i = sum_j g_ij dA_ij / sum_j g_ij,
 *   dS_ij = g_ij (dA_ij - delta_i),
 *   dQ = scale dS K,  dK = scale dS^T Q,  dV = A^T dO.
 *   Q, K, V, dO  [B][H][L][d] of `dtype`; tau and block_mask exactly as
 *   written by entmax_attn_fwd for the same Q, K, V, scale, mask, window.
 *   dQ, dK, dV   [B][H][L][d] fp32 outputs (overwritten).
 *   workspace    at least entmax_attn_bwd_workspace(...) bytes.
 * For bf16 inputs the products with A and dS take fp16 operands scaled by
 * powers of two, so any finite input range is handled; Q, K, V, dO must be
 * finite.
 */
int entmax_attn_bwd(const void* Q, const void* K, const void* V, const void* dO,
                    const float* tau, const uint32_t* block_mask, float* dQ, float* dK,
                    float* dV, int B, int H, int L, int d, float scale, float alpha,
                    int dtype, int mask, int window, void* workspace,
                    size_t workspace_bytes, void* stream);

/*
 * Forward and backward for training, without the backward's delta pass.
 *
 * delta_i = sum_j g_ij dA_ij / sum_j g_ij (g_ij = dA_ij/dS_ij, the derivative
 * of the weights in the scores: [(S_ij - tau_i)/2]_+ at alpha = 1.5, and
 * [(alpha-1)(S_ij - tau_i)]_+^(1/(alpha-1) - 1) otherwise; dA_ij = dO_i . V_j)
 * equals dO_i . GV_i / gsum_i with GV_i = sum_j g_ij V_j and
 * gsum_i = sum_j g_ij.  The threshold's implicit derivative on the support
 * ("AdaSplash-2: Faster Differentiable Sparse Attention", sec. 3.3 "Backward
 * pass") needs delta; entmax_attn_bwd gets it from an extra pass over every
 * row's non-null tiles, which these two calls replace by one more product in
 * the forward's output phase and a dot product per row.
 *
 * entmax_attn_fwd_gv: entmax_attn_fwd (same arguments, workspace and
 *   results: O, tau and the mask are bit-identical) that also writes
 *     GV    [B][H][L][d] fp32, 16-byte aligned (overwritten)
 *     gsum  [B][H][L] fp32 (overwritten)
 * entmax_attn_bwd_gv: entmax_attn_bwd (same arguments and workspace) that
 *   takes GV and gsum from entmax_attn_fwd_gv on the same inputs.
 * Both need bf16 inputs (ENTMAX_ERR_DTYPE otherwise) and L <= 16384
 * (ENTMAX_ERR_SHAPE otherwise); NULL GV or gsum is ENTMAX_ERR_NULL.
 */
int entmax_attn_fwd_gv(const void* Q, const void* K, const void* V, float* O, float* tau,
                       uint32_t* block_mask, float* GV, float* gsum, int B, int H, int L, int d,
                       float scale, float alpha, int dtype, int mask, int window, void* workspace,
                       size_t workspace_bytes, void* stream);
int entmax_attn_bwd_gv(const void* Q, const void* K, const void* V, const void* dO,
                       const float* tau, const uint32_t* block_mask, const float* GV,
                       const float* gsum, float* dQ, float* dK, float* dV, int B, int H, int L,
                       int d, float scale, float alpha, int dtype, int mask, int window,
                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * One decode step: the newest query of every (batch, head), at position
 * L - 1, against the first L rows of its KV cache.  Exactly the last query
 * row of entmax_attn_fwd for the same mask mode (mode 0 and mode 1 both
 * attend to every cached key; mode 2 to key 0 and the keys at most `window`
 * positions behind).  Autoregressive generation over a growing cache is the
 * setting of "GPT-2 with AdaSplash Attention via NeuralOps" (Architecture
 * Overview; Mathematical Formulation item 1); "AdaSplash-2: Faster
 * Differentiable Sparse Attention" sec. 5 leaves an inference kernel to
 * future work.  Only the support's V rows are read (the block traversal of
 * AdaSplash-2 sec. 3.3 phase 4 at single-key granularity).
 *   q        [B][H][d] of `dtype`, 16-byte aligned.
 *   K, V     caches [B][H][cache_len][d] of `dtype`, 16-byte aligned; rows
 *            0 .. L - 1 are read, L <= cache_len.
 *   O        [B][H][d] fp32 output;  tau  [B][H] fp32 output (score units).
 *   d in {64, 128}; 1 <= L <= 2^24; B * H <= 65535; alpha in (1, 2].
 *   workspace  at least entmax_attn_decode_workspace(B, H, L, d, dtype,
 *              mask, window) bytes (4 bytes per active key per head).
 * Returns the codes of entmax_attn_fwd.
 */
size_t entmax_attn_decode_workspace(int B, int H, int L, int d, int dtype, int mask,
                                    int window);
int entmax_attn_decode(const void* q, const void* K, const void* V, float* O, float* tau,
                       int B, int H, int L, int cache_len, int d, float scale, float alpha,
                       int dtype, int mask, int window, void* workspace,
                       size_t workspace_bytes, void* stream);

/*
 * entmax_attn_decode without a workspace, for callers that cannot allocate
 * device memory around the call: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  Same arguments, results and error
 * codes as entmax_attn_decode, minus the workspace pair; it calls no
 * allocating routine.  The per-key scores go to a static scratch array of
 * ENTMAX_DECODE_SCRATCH_BYTES bytes that each device holds until the process
 * ends: B * H * (active keys per head) * 4 bytes must fit in it (8,388,608
 * active keys over all heads; e.g. B * H = 256 heads of 32768 cached keys),
 * else ENTMAX_ERR_SCRATCH before any launch.  Every call on one device
 * shares that device's scratch: calls that overlap on one device (different
 * streams, different threads) race and must be serialised by the caller.
 * Nothing in the scratch needs clearing between calls (each call writes the
 * scores before reading them).
 */
#define ENTMAX_DECODE_SCRATCH_BYTES ((size_t)32 << 20)
int entmax_attn_decode_noalloc(const void* q, const void* K, const void* V, float* O, float* tau,
                               int B, int H, int L, int cache_len, int d, float scale, float alpha,
                               int dtype, int mask, int window, void* stream);

/*
 * Per-call options of the _ex entry points below.  A zero-initialised struct
 * (or a NULL pointer) selects the defaults, which are what the plain entry
 * points use.
 *  candidate_cap: per-row capacity of the forward's candidate list, 1 .. 128
 *    (0: 128).  Rows with more candidates above their lower bound take the
 *    histogram-initialised sweeps (AdaSplash-2 sec. 3.1 and sec. 3.3 phases
 *    2-3); tests use a tiny cap to force that path.  Results agree either way
 *    within the tolerances.  Values outside 0 .. 128 give ENTMAX_ERR_ARG.
 *  row_plain_bracket: entmax_tau_rows on rows that it streams from memory
 *    (wider than 32768, or wider than 8192 without 16-byte row alignment)
 *    starts its refinement from the histogram bracket
 *    [tau_h, tau_h + 1/(64 (alpha-1))] of AdaSplash-2 sec. 3.1 and
 *    Proposition 3.1 (0, the default), or from the plain bracket
 *    [m - 1/(alpha-1), m - n^(1-alpha)/(alpha-1)] (1).  Rows it holds in
 *    registers always start from the plain bracket (a refinement step over
 *    registers costs less than building the histogram).  Other values give
 *    ENTMAX_ERR_ARG.
 */
typedef struct entmax_options {
    int candidate_cap;
    int row_plain_bracket;
} entmax_options;

int entmax_tau_rows_ex(const float* S, float* P, float* tau, int64_t rows, int64_t cols,
                       int64_t ld, float alpha, const entmax_options* options, void* stream);
int entmax_attn_fwd_ex(const void* Q, const void* K, const void* V, float* O, float* tau,
                       uint32_t* block_mask, int B, int H, int L, int d, float scale, float alpha,
                       int dtype, int mask, int window, void* workspace, size_t workspace_bytes,
                       const entmax_options* options, void* stream);
int entmax_attn_threshold_ex(const void* Q, const void* K, float* tau, uint32_t* block_mask,
                             int B, int H, int L, int d, float scale, float alpha, int dtype,
                             int mask, int window, void* workspace, size_t workspace_bytes,
                             const entmax_options* options, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* ENTMAX_H */
