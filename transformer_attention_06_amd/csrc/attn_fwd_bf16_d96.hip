// attn_fwd_bf16_d96.hip — the __bf16, D = 96 instances of the fused attention
// forward kernel (attn_fwd_kernel.h; LDS rows of 128 dims, the slots past
// 96 zero); one translation unit per element type and head dim.
#include "attn_fwd_kernel.h"

namespace attn_detail {

int launch_fwd_bf16_d96(const LaunchArgs& a) { return launch_d_plain<__bf16, 96>(a); }

}  // namespace attn_detail
