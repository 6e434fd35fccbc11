// launch.hpp -- internal launchers behind the C ABI (not exported).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace entmax {

// use_hist: histogram-initialised bracket in the wide-row kernel
hipError_t launch_tau_rows(const float* S, float* P, float* tau, int64_t rows, int64_t cols,
                           int64_t ld, float alpha, int use_hist, hipStream_t stream);

// Arguments of one attention call after validation.
struct AttnArgs {
    const void* q;
    const void* k;
    const void* v;
    const void* dout;      // backward only
    float* o;              // forward only
    float* tau;            // forward writes, backward reads
    uint32_t* block_mask;  // forward writes (may be null); backward reads
    float* dq;
    float* dk;
    float* dv;
    float* gv;    // forward writes (may be null), backward reads (null: delta pass)
    float* gsum;  // same
    int B, H, L, d;
    float scale;
    float alpha;  // in (1, 2]
    int dtype;  // 0 fp32, 1 bf16
    int mask;   // 0 none, 1 causal, 2 causal window + sink
    int window;
    int cand_cap;  // forward candidate capacity per row
    void* workspace;
    size_t workspace_bytes;
};

// Block-mask tile (rows x cols) of the forward.
constexpr int kMaskBr = 64;
constexpr int kMaskBc = 64;

size_t attn_threshold_workspace_bytes(int B, int H, int L);
size_t attn_fwd_workspace_bytes(int B, int H, int L, int d, int dtype);
size_t attn_bwd_workspace_bytes(int B, int H, int L, int d, int dtype);
int attn_max_candidate_cap(int d, int dtype);
// phase bits: 1 = score statistics, 2 = threshold solve + mask, 4 = output
hipError_t launch_attn_fwd(const AttnArgs& a, int phase, hipStream_t stream);
hipError_t launch_attn_bwd(const AttnArgs& a, hipStream_t stream);
// Decode step: a.q is [B][H][d] (the query at position L - 1), a.k / a.v the
// caches [B][H][Lcap][d] of which rows 0 .. L - 1 are used; a.o [B][H][d].
size_t attn_decode_workspace_bytes(int B, int H, int L, int mask, int window);
hipError_t launch_attn_decode(const AttnArgs& a, int Lcap, hipStream_t stream);
// Bytes of the static per-device scratch of the allocation-free decode, and
// its device address on the current device (looked up once per device).
constexpr size_t kDecodeScratchBytes = (size_t)32 << 20;
hipError_t decode_scratch_address(void** out);

}  // namespace entmax
