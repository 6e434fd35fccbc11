// attn_bwd.hip -- placeholder until the backward kernels land.
#include "launch.hpp"
namespace entmax {
size_t attn_bwd_workspace_bytes(int B, int H, int L, int, int) {
    return ((size_t)B * H * L * 2 * sizeof(float) + 255) & ~(size_t)255;
}
hipError_t launch_attn_bwd(const AttnArgs&, hipStream_t) { return hipErrorNotSupported; }
}  // namespace entmax
