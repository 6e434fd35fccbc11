// entmax_api.cpp -- the exported C ABI: argument validation, then launches.
// Declarations and the contract of every entry point are in include/entmax.h.
#include "../../include/entmax.h"

#include <hip/hip_runtime.h>
#include <math.h>

#include "launch.hpp"

namespace {

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int hip_status(hipError_t e) { return e == hipSuccess ? ENTMAX_OK : ENTMAX_ERR_HIP; }

// Options of one call (NULL: defaults); ENTMAX_ERR_ARG for values out of range.
int read_options(const entmax_options* o, int* cand_cap, int* row_hist) {
    *cand_cap = 0;
    *row_hist = 1;
    if (o == nullptr) return ENTMAX_OK;
    if (o->candidate_cap < 0 || o->candidate_cap > entmax::attn_max_candidate_cap(64, ENTMAX_BF16))
        return ENTMAX_ERR_ARG;
    if (o->row_plain_bracket != 0 && o->row_plain_bracket != 1) return ENTMAX_ERR_ARG;
    *cand_cap = o->candidate_cap;
    *row_hist = o->row_plain_bracket ? 0 : 1;
    return ENTMAX_OK;
}

// Shared checks of the attention entry points (everything except pointers).
// Longest sequence of the fused forward kernel, the only one that writes G.V.
constexpr int kGvMaxL = 16384;

int check_attn_shape(int B, int H, int L, int d, float alpha, int dtype, int mask, int window) {
    if (!(alpha > 1.0f && alpha <= 2.0f)) return ENTMAX_ERR_ALPHA;
    if (dtype != ENTMAX_F32 && dtype != ENTMAX_BF16) return ENTMAX_ERR_DTYPE;
    if (mask != ENTMAX_MASK_NONE && mask != ENTMAX_MASK_CAUSAL &&
        mask != ENTMAX_MASK_CAUSAL_WINDOW_SINK)
        return ENTMAX_ERR_MASK;
    if (mask == ENTMAX_MASK_CAUSAL_WINDOW_SINK && window < 0) return ENTMAX_ERR_MASK;
    if (B < 1 || H < 1 || L < 1 || (d != 64 && d != 128)) return ENTMAX_ERR_SHAPE;
    if ((int64_t)B * H > 0x7fffffffLL || L > (1 << 16) ||
        (int64_t)B * H * L * d > (int64_t)1 << 40)
        return ENTMAX_ERR_SHAPE;
    return ENTMAX_OK;
}

}  // namespace

extern "C" {

const char* entmax_status_str(int status) {
    switch (status) {
        case ENTMAX_OK: return "ok";
        case ENTMAX_ERR_NULL: return "null pointer argument";
        case ENTMAX_ERR_SHAPE: return "unsupported or inconsistent shape";
        case ENTMAX_ERR_ALPHA: return "alpha must lie in (1, 2]";
        case ENTMAX_ERR_DTYPE: return "unknown dtype";
        case ENTMAX_ERR_MASK: return "unknown mask mode or negative window";
        case ENTMAX_ERR_WORKSPACE: return "workspace missing or too small";
        case ENTMAX_ERR_ALIGN: return "pointer not 16-byte aligned";
        case ENTMAX_ERR_HIP: return "HIP launch failed";
        case ENTMAX_ERR_ARG: return "invalid argument";
        case ENTMAX_ERR_SCRATCH: return "input exceeds the static scratch of the allocation-free entry point";
        default: return "unknown status";
    }
}

int entmax_version(void) { return (1 << 16) | 0; }

int entmax_tile_shape(int d, int dtype, int* block_rows, int* block_cols) {
    if (block_rows == nullptr || block_cols == nullptr) return ENTMAX_ERR_NULL;
    if (dtype != ENTMAX_F32 && dtype != ENTMAX_BF16) return ENTMAX_ERR_DTYPE;
    if (d != 64 && d != 128) return ENTMAX_ERR_SHAPE;
    *block_rows = entmax::kMaskBr;
    *block_cols = entmax::kMaskBc;
    return ENTMAX_OK;
}

int entmax_tau_rows_ex(const float* S, float* P, float* tau, int64_t rows, int64_t cols,
                       int64_t ld, float alpha, const entmax_options* options, void* stream) {
    if (!(alpha > 1.0f && alpha <= 2.0f)) return ENTMAX_ERR_ALPHA;
    if (rows < 0 || cols < 1 || ld < cols || rows > 0x7fffffffLL || cols > 0x7fffffffLL)
        return ENTMAX_ERR_SHAPE;
    int cap, row_hist;
    const int st = read_options(options, &cap, &row_hist);
    if (st != ENTMAX_OK) return st;
    if (rows == 0) return ENTMAX_OK;
    if (S == nullptr || tau == nullptr) return ENTMAX_ERR_NULL;
    (void)hipGetLastError();
    return hip_status(
        entmax::launch_tau_rows(S, P, tau, rows, cols, ld, alpha, row_hist, (hipStream_t)stream));
}

int entmax_tau_rows(const float* S, float* P, float* tau, int64_t rows, int64_t cols,
                    int64_t ld, float alpha, void* stream) {
    return entmax_tau_rows_ex(S, P, tau, rows, cols, ld, alpha, nullptr, stream);
}

size_t entmax_attn_threshold_workspace(int B, int H, int L, int d, int dtype, int mask,
                                       int window) {
    if (check_attn_shape(B, H, L, d, 1.5f, dtype, mask, window) != ENTMAX_OK) return 0;
    return entmax::attn_threshold_workspace_bytes(B, H, L);
}

size_t entmax_attn_fwd_workspace(int B, int H, int L, int d, int dtype, int mask, int window) {
    if (check_attn_shape(B, H, L, d, 1.5f, dtype, mask, window) != ENTMAX_OK) return 0;
    return entmax::attn_fwd_workspace_bytes(B, H, L, d, dtype);
}

}  // extern "C"

namespace {

// The forward, with G.V and sum g as well when gv is not null (bf16, the
// fused kernel's range of L only).
int attn_fwd_impl(const void* Q, const void* K, const void* V, float* O, float* tau,
                  uint32_t* block_mask, float* gv, float* gsum, int B, int H, int L, int d, float scale,
                  float alpha, int dtype, int mask, int window, void* workspace, size_t workspace_bytes,
                  const entmax_options* options, void* stream) {
    if (Q == nullptr || K == nullptr || V == nullptr || O == nullptr || tau == nullptr)
        return ENTMAX_ERR_NULL;
    int st = check_attn_shape(B, H, L, d, alpha, dtype, mask, window);
    if (st != ENTMAX_OK) return st;
    if (!(scale > 0.0f) || !isfinite(scale)) return ENTMAX_ERR_ARG;
    if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O)) return ENTMAX_ERR_ALIGN;
    if (((uintptr_t)tau & 3u) || ((uintptr_t)block_mask & 3u)) return ENTMAX_ERR_ALIGN;
    const size_t need = block_mask ? entmax::attn_threshold_workspace_bytes(B, H, L)
                                   : entmax::attn_fwd_workspace_bytes(B, H, L, d, dtype);
    if (workspace == nullptr || workspace_bytes < need) return ENTMAX_ERR_WORKSPACE;
    if (!aligned16(workspace)) return ENTMAX_ERR_ALIGN;
    int cap, row_hist;
    st = read_options(options, &cap, &row_hist);
    if (st != ENTMAX_OK) return st;
    entmax::AttnArgs a = {};
    a.q = Q; a.k = K; a.v = V; a.o = O; a.tau = tau; a.block_mask = block_mask;
    a.B = B; a.H = H; a.L = L; a.d = d; a.scale = scale; a.alpha = alpha; a.dtype = dtype;
    a.mask = mask; a.window = mask == ENTMAX_MASK_CAUSAL_WINDOW_SINK ? window : 0;
    const int maxcap = entmax::attn_max_candidate_cap(d, dtype);
    a.cand_cap = (cap > 0 && cap < maxcap) ? cap : maxcap;
    a.workspace = workspace; a.workspace_bytes = workspace_bytes;
    a.gv = gv; a.gsum = gsum;
    (void)hipGetLastError();
    return hip_status(entmax::launch_attn_fwd(a, 7, (hipStream_t)stream));
}

// The backward; with gv and gsum from the forward, delta comes from them
// instead of a pass over the keys (bf16 only).
int attn_bwd_impl(const void* Q, const void* K, const void* V, const void* dO, const float* tau,
                  const uint32_t* block_mask, const float* gv, const float* gsum, float* dQ, float* dK,
                  float* dV, int B, int H, int L, int d, float scale, float alpha, int dtype, int mask,
                  int window, void* workspace, size_t workspace_bytes, void* stream);

}  // namespace

extern "C" {

int entmax_attn_fwd_ex(const void* Q, const void* K, const void* V, float* O, float* tau,
                       uint32_t* block_mask, int B, int H, int L, int d, float scale, float alpha,
                       int dtype, int mask, int window, void* workspace, size_t workspace_bytes,
                       const entmax_options* options, void* stream) {
    return attn_fwd_impl(Q, K, V, O, tau, block_mask, nullptr, nullptr, B, H, L, d, scale, alpha, dtype,
                         mask, window, workspace, workspace_bytes, options, stream);
}

int entmax_attn_fwd_gv(const void* Q, const void* K, const void* V, float* O, float* tau,
                       uint32_t* block_mask, float* GV, float* gsum, int B, int H, int L, int d,
                       float scale, float alpha, int dtype, int mask, int window, void* workspace,
                       size_t workspace_bytes, void* stream) {
    if (GV == nullptr || gsum == nullptr) return ENTMAX_ERR_NULL;
    int st = check_attn_shape(B, H, L, d, alpha, dtype, mask, window);
    if (st != ENTMAX_OK) return st;
    if (dtype != ENTMAX_BF16) return ENTMAX_ERR_DTYPE;
    if (L > kGvMaxL) return ENTMAX_ERR_SHAPE;
    if (!aligned16(GV) || ((uintptr_t)gsum & 3u)) return ENTMAX_ERR_ALIGN;
    return attn_fwd_impl(Q, K, V, O, tau, block_mask, GV, gsum, B, H, L, d, scale, alpha, dtype, mask,
                         window, workspace, workspace_bytes, nullptr, stream);
}

int entmax_attn_fwd(const void* Q, const void* K, const void* V, float* O, float* tau,
                    uint32_t* block_mask, int B, int H, int L, int d, float scale, float alpha,
                    int dtype, int mask, int window, void* workspace, size_t workspace_bytes,
                    void* stream) {
    return entmax_attn_fwd_ex(Q, K, V, O, tau, block_mask, B, H, L, d, scale, alpha, dtype, mask,
                              window, workspace, workspace_bytes, nullptr, stream);
}

int entmax_attn_threshold_ex(const void* Q, const void* K, float* tau, uint32_t* block_mask,
                             int B, int H, int L, int d, float scale, float alpha, int dtype,
                             int mask, int window, void* workspace, size_t workspace_bytes,
                             const entmax_options* options, void* stream) {
    if (Q == nullptr || K == nullptr || tau == nullptr || block_mask == nullptr)
        return ENTMAX_ERR_NULL;
    int st = check_attn_shape(B, H, L, d, alpha, dtype, mask, window);
    if (st != ENTMAX_OK) return st;
    if (!(scale > 0.0f) || !isfinite(scale)) return ENTMAX_ERR_ARG;
    if (!aligned16(Q) || !aligned16(K)) return ENTMAX_ERR_ALIGN;
    if (((uintptr_t)tau & 3u) || ((uintptr_t)block_mask & 3u)) return ENTMAX_ERR_ALIGN;
    if (workspace == nullptr || workspace_bytes < entmax::attn_threshold_workspace_bytes(B, H, L))
        return ENTMAX_ERR_WORKSPACE;
    if (!aligned16(workspace)) return ENTMAX_ERR_ALIGN;
    int cap, row_hist;
    st = read_options(options, &cap, &row_hist);
    if (st != ENTMAX_OK) return st;
    entmax::AttnArgs a = {};
    a.q = Q; a.k = K; a.tau = tau; a.block_mask = block_mask;
    a.workspace = workspace; a.workspace_bytes = workspace_bytes;
    a.B = B; a.H = H; a.L = L; a.d = d; a.scale = scale; a.alpha = alpha; a.dtype = dtype;
    a.mask = mask; a.window = mask == ENTMAX_MASK_CAUSAL_WINDOW_SINK ? window : 0;
    const int maxcap = entmax::attn_max_candidate_cap(d, dtype);
    a.cand_cap = (cap > 0 && cap < maxcap) ? cap : maxcap;
    (void)hipGetLastError();
    return hip_status(entmax::launch_attn_fwd(a, 3, (hipStream_t)stream));
}

int entmax_attn_threshold(const void* Q, const void* K, float* tau, uint32_t* block_mask,
                          int B, int H, int L, int d, float scale, float alpha, int dtype,
                          int mask, int window, void* workspace, size_t workspace_bytes,
                          void* stream) {
    return entmax_attn_threshold_ex(Q, K, tau, block_mask, B, H, L, d, scale, alpha, dtype, mask,
                                    window, workspace, workspace_bytes, nullptr, stream);
}

int entmax_attn_score_stats(const void* Q, const void* K, int B, int H, int L, int d, float scale,
                            float alpha, int dtype, int mask, int window, void* workspace,
                            size_t workspace_bytes, void* stream) {
    if (Q == nullptr || K == nullptr) return ENTMAX_ERR_NULL;
    int st = check_attn_shape(B, H, L, d, alpha, dtype, mask, window);
    if (st != ENTMAX_OK) return st;
    if (!(scale > 0.0f) || !isfinite(scale)) return ENTMAX_ERR_ARG;
    if (!aligned16(Q) || !aligned16(K)) return ENTMAX_ERR_ALIGN;
    if (workspace == nullptr || workspace_bytes < entmax::attn_threshold_workspace_bytes(B, H, L))
        return ENTMAX_ERR_WORKSPACE;
    if (!aligned16(workspace)) return ENTMAX_ERR_ALIGN;
    entmax::AttnArgs a = {};
    a.q = Q; a.k = K;
    a.B = B; a.H = H; a.L = L; a.d = d; a.scale = scale; a.alpha = alpha; a.dtype = dtype;
    a.mask = mask; a.window = mask == ENTMAX_MASK_CAUSAL_WINDOW_SINK ? window : 0;
    a.workspace = workspace; a.workspace_bytes = workspace_bytes;
    (void)hipGetLastError();
    return hip_status(entmax::launch_attn_fwd(a, 1, (hipStream_t)stream));
}

int entmax_attn_output(const void* Q, const void* K, const void* V, const float* tau,
                       const uint32_t* block_mask, float* O, int B, int H, int L, int d,
                       float scale, float alpha, int dtype, int mask, int window,
                       void* stream) {
    if (Q == nullptr || K == nullptr || V == nullptr || tau == nullptr ||
        block_mask == nullptr || O == nullptr)
        return ENTMAX_ERR_NULL;
    int st = check_attn_shape(B, H, L, d, alpha, dtype, mask, window);
    if (st != ENTMAX_OK) return st;
    if (!(scale > 0.0f) || !isfinite(scale)) return ENTMAX_ERR_ARG;
    if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O)) return ENTMAX_ERR_ALIGN;
    if (((uintptr_t)tau & 3u) || ((uintptr_t)block_mask & 3u)) return ENTMAX_ERR_ALIGN;
    entmax::AttnArgs a = {};
    a.q = Q; a.k = K; a.v = V; a.o = O; a.tau = const_cast<float*>(tau);
    a.block_mask = const_cast<uint32_t*>(block_mask);
    a.B = B; a.H = H; a.L = L; a.d = d; a.scale = scale; a.alpha = alpha; a.dtype = dtype;
    a.mask = mask; a.window = mask == ENTMAX_MASK_CAUSAL_WINDOW_SINK ? window : 0;
    (void)hipGetLastError();
    return hip_status(entmax::launch_attn_fwd(a, 4, (hipStream_t)stream));
}

size_t entmax_attn_bwd_workspace(int B, int H, int L, int d, int dtype, int mask, int window) {
    if (check_attn_shape(B, H, L, d, 1.5f, dtype, mask, window) != ENTMAX_OK) return 0;
    return entmax::attn_bwd_workspace_bytes(B, H, L, d, dtype);
}

int entmax_attn_bwd(const void* Q, const void* K, const void* V, const void* dO,
                    const float* tau, const uint32_t* block_mask, float* dQ, float* dK,
                    float* dV, int B, int H, int L, int d, float scale, float alpha, int dtype,
                    int mask, int window, void* workspace, size_t workspace_bytes,
                    void* stream) {
    return attn_bwd_impl(Q, K, V, dO, tau, block_mask, nullptr, nullptr, dQ, dK, dV, B, H, L, d, scale, alpha,
                         dtype, mask, window, workspace, workspace_bytes, stream);
}

int entmax_attn_bwd_gv(const void* Q, const void* K, const void* V, const void* dO,
                       const float* tau, const uint32_t* block_mask, const float* GV,
                       const float* gsum, float* dQ, float* dK, float* dV, int B, int H, int L,
                       int d, float scale, float alpha, int dtype, int mask, int window,
                       void* workspace, size_t workspace_bytes, void* stream) {
    if (GV == nullptr || gsum == nullptr) return ENTMAX_ERR_NULL;
    int st = check_attn_shape(B, H, L, d, alpha, dtype, mask, window);
    if (st != ENTMAX_OK) return st;
    if (dtype != ENTMAX_BF16) return ENTMAX_ERR_DTYPE;
    if (L > kGvMaxL) return ENTMAX_ERR_SHAPE;
    if (!aligned16(GV) || ((uintptr_t)gsum & 3u)) return ENTMAX_ERR_ALIGN;
    return attn_bwd_impl(Q, K, V, dO, tau, block_mask, GV, gsum, dQ, dK, dV, B, H, L, d, scale, alpha, dtype,
                         mask, window, workspace, workspace_bytes, stream);
}

}  // extern "C"

namespace {

int attn_bwd_impl(const void* Q, const void* K, const void* V, const void* dO, const float* tau,
                  const uint32_t* block_mask, const float* gv, const float* gsum, float* dQ, float* dK,
                  float* dV, int B, int H, int L, int d, float scale, float alpha, int dtype, int mask,
                  int window, void* workspace, size_t workspace_bytes, void* stream) {
    if (Q == nullptr || K == nullptr || V == nullptr || dO == nullptr || tau == nullptr ||
        block_mask == nullptr || dQ == nullptr || dK == nullptr || dV == nullptr)
        return ENTMAX_ERR_NULL;
    int st = check_attn_shape(B, H, L, d, alpha, dtype, mask, window);
    if (st != ENTMAX_OK) return st;
    if (!(scale > 0.0f) || !isfinite(scale)) return ENTMAX_ERR_ARG;
    if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(dO) || !aligned16(dQ) ||
        !aligned16(dK) || !aligned16(dV))
        return ENTMAX_ERR_ALIGN;
    if (((uintptr_t)tau & 3u) || ((uintptr_t)block_mask & 3u)) return ENTMAX_ERR_ALIGN;
    const size_t need = entmax::attn_bwd_workspace_bytes(B, H, L, d, dtype);
    if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return ENTMAX_ERR_WORKSPACE;
    if (need > 0 && !aligned16(workspace)) return ENTMAX_ERR_ALIGN;
    entmax::AttnArgs a = {};
    a.q = Q; a.k = K; a.v = V; a.dout = dO; a.tau = const_cast<float*>(tau);
    a.block_mask = const_cast<uint32_t*>(block_mask);
    a.dq = dQ; a.dk = dK; a.dv = dV;
    a.gv = const_cast<float*>(gv); a.gsum = const_cast<float*>(gsum);
    a.B = B; a.H = H; a.L = L; a.d = d; a.scale = scale; a.alpha = alpha; a.dtype = dtype;
    a.mask = mask; a.window = mask == ENTMAX_MASK_CAUSAL_WINDOW_SINK ? window : 0;
    a.workspace = workspace; a.workspace_bytes = workspace_bytes;
    (void)hipGetLastError();
    return hip_status(entmax::launch_attn_bwd(a, (hipStream_t)stream));
}

}  // namespace

namespace {
constexpr int kMaxDecodeLen = 1 << 24;

int check_decode(int B, int H, int L, int Lcap, int d, float alpha, int dtype, int mask,
                 int window) {
    if (!(alpha > 1.0f && alpha <= 2.0f)) return ENTMAX_ERR_ALPHA;
    if (dtype != ENTMAX_F32 && dtype != ENTMAX_BF16) return ENTMAX_ERR_DTYPE;
    if (mask != ENTMAX_MASK_NONE && mask != ENTMAX_MASK_CAUSAL &&
        mask != ENTMAX_MASK_CAUSAL_WINDOW_SINK)
        return ENTMAX_ERR_MASK;
    if (mask == ENTMAX_MASK_CAUSAL_WINDOW_SINK && window < 0) return ENTMAX_ERR_MASK;
    if (B < 1 || H < 1 || L < 1 || Lcap < L || L > kMaxDecodeLen || (d != 64 && d != 128))
        return ENTMAX_ERR_SHAPE;
    if ((int64_t)B * H > 65535 || (int64_t)B * H * Lcap * d > (int64_t)1 << 40)
        return ENTMAX_ERR_SHAPE;
    return ENTMAX_OK;
}
}  // namespace

extern "C" {

size_t entmax_attn_decode_workspace(int B, int H, int L, int d, int dtype, int mask, int window) {
    if (check_decode(B, H, L, L, d, 1.5f, dtype, mask, window) != ENTMAX_OK) return 0;
    return entmax::attn_decode_workspace_bytes(B, H, L, mask, window);
}

int entmax_attn_decode(const void* q, const void* K, const void* V, float* O, float* tau,
                       int B, int H, int L, int cache_len, int d, float scale, float alpha,
                       int dtype, int mask, int window, void* workspace, size_t workspace_bytes,
                       void* stream) {
    if (q == nullptr || K == nullptr || V == nullptr || O == nullptr || tau == nullptr)
        return ENTMAX_ERR_NULL;
    int st = check_decode(B, H, L, cache_len, d, alpha, dtype, mask, window);
    if (st != ENTMAX_OK) return st;
    if (!(scale > 0.0f) || !isfinite(scale)) return ENTMAX_ERR_ARG;
    if (!aligned16(q) || !aligned16(K) || !aligned16(V)) return ENTMAX_ERR_ALIGN;
    if (((uintptr_t)O & 3u) || ((uintptr_t)tau & 3u)) return ENTMAX_ERR_ALIGN;
    const size_t need = entmax::attn_decode_workspace_bytes(B, H, L, mask, window);
    if (workspace == nullptr || workspace_bytes < need) return ENTMAX_ERR_WORKSPACE;
    if ((uintptr_t)workspace & 3u) return ENTMAX_ERR_ALIGN;
    entmax::AttnArgs a = {};
    a.q = q; a.k = K; a.v = V; a.o = O; a.tau = tau;
    a.B = B; a.H = H; a.L = L; a.d = d; a.scale = scale; a.alpha = alpha; a.dtype = dtype;
    a.mask = mask; a.window = mask == ENTMAX_MASK_CAUSAL_WINDOW_SINK ? window : 0;
    a.workspace = workspace; a.workspace_bytes = workspace_bytes;
    (void)hipGetLastError();
    return hip_status(entmax::launch_attn_decode(a, cache_len, (hipStream_t)stream));
}

}  // extern "C"

extern "C" {

int entmax_attn_decode_noalloc(const void* q, const void* K, const void* V, float* O, float* tau,
                               int B, int H, int L, int cache_len, int d, float scale, float alpha,
                               int dtype, int mask, int window, void* stream) {
    if (q == nullptr || K == nullptr || V == nullptr || O == nullptr || tau == nullptr)
        return ENTMAX_ERR_NULL;
    int st = check_decode(B, H, L, cache_len, d, alpha, dtype, mask, window);
    if (st != ENTMAX_OK) return st;
    if (!(scale > 0.0f) || !isfinite(scale)) return ENTMAX_ERR_ARG;
    if (!aligned16(q) || !aligned16(K) || !aligned16(V)) return ENTMAX_ERR_ALIGN;
    if (((uintptr_t)O & 3u) || ((uintptr_t)tau & 3u)) return ENTMAX_ERR_ALIGN;
    if (entmax::attn_decode_workspace_bytes(B, H, L, mask, window) > entmax::kDecodeScratchBytes)
        return ENTMAX_ERR_SCRATCH;
    void* scratch = nullptr;
    (void)hipGetLastError();
    if (entmax::decode_scratch_address(&scratch) != hipSuccess) return ENTMAX_ERR_HIP;
    entmax::AttnArgs a = {};
    a.q = q; a.k = K; a.v = V; a.o = O; a.tau = tau;
    a.B = B; a.H = H; a.L = L; a.d = d; a.scale = scale; a.alpha = alpha; a.dtype = dtype;
    a.mask = mask; a.window = mask == ENTMAX_MASK_CAUSAL_WINDOW_SINK ? window : 0;
    a.workspace = scratch; a.workspace_bytes = entmax::kDecodeScratchBytes;
    return hip_status(entmax::launch_attn_decode(a, cache_len, (hipStream_t)stream));
}

}  // extern "C"
