// attn_fwd_f16_d112.hip — the _Float16, D = 112 instances of the fused attention
// forward kernel (attn_fwd_kernel.h; LDS rows of 128 dims, the slots past
// 112 zero); one translation unit per element type and head dim.
#include "attn_fwd_kernel.h"

namespace attn_detail {

int launch_fwd_f16_d112(const LaunchArgs& a) { return launch_d_plain<_Float16, 112>(a); }

}  // namespace attn_detail
