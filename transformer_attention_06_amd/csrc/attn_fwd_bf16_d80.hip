// attn_fwd_bf16_d80.hip — the __bf16, D = 80 instances of the fused attention
// forward kernel (attn_fwd_kernel.h; LDS rows of 128 dims, the slots past
// 80 zero); one translation unit per element type and head dim.
#include "attn_fwd_kernel.h"

namespace attn_detail {

int launch_fwd_bf16_d80(const LaunchArgs& a) { return launch_d_plain<__bf16, 80>(a); }

}  // namespace attn_detail
