// attn_fwd_bf16_d256.hip — the __bf16, D = 256 instances of the fused attention
// forward kernel (attn_fwd_kernel.h; 32-key tiles, LDS rows of 256 dims, one
// wavefront per SIMD with the output accumulators in AGPRs); one
// translation unit per element type and head dim.
#include "attn_fwd_kernel.h"

namespace attn_detail {

int launch_fwd_bf16_d256(const LaunchArgs& a) { return launch_d_plain<__bf16, 256>(a); }

}  // namespace attn_detail
