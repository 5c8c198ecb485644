// Replay-attention backward on gfx950 bf16 matrix cores (placeholder: generic kernels).
#include "common.hpp"
#include "launch.hpp"

namespace ls {

hipError_t launch_bwd_mfma(const AttnArgs& a, hipStream_t s) { return launch_bwd_generic(1, a, s); }

}  // namespace ls
