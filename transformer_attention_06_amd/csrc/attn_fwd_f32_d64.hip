// attn_fwd_f32_d64.hip — the float, D = 64 instances of the fused attention
// forward kernel (attn_fwd_kernel.h); one translation unit per element type
// and head dim, so the instances compile in parallel.
#include "attn_fwd_kernel.h"

namespace attn_detail {

int launch_fwd_f32_d64(const LaunchArgs& a) { return launch_d<float, 64>(a); }

}  // namespace attn_detail
