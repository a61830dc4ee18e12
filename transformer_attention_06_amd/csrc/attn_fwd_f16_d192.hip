// attn_fwd_f16_d192.hip — the _Float16, D = 192 instances of the fused attention
// forward kernel (attn_fwd_kernel.h; 32-key tiles, LDS rows of 256 dims, one
// wavefront per SIMD with the output accumulators in AGPRs); one
// translation unit per element type and head dim.
#include "attn_fwd_kernel.h"

namespace attn_detail {

int launch_fwd_f16_d192(const LaunchArgs& a) { return launch_d_plain<_Float16, 192>(a); }

}  // namespace attn_detail
