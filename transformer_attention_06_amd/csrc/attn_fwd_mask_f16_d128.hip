// attn_fwd_mask_f16_d128.hip — the _Float16, D = 128 instances of the fused
// attention forward kernel (attn_fwd_kernel.h) with a mask tensor.
#include "attn_fwd_kernel.h"

namespace attn_detail {

int launch_fwd_mask_f16_d128(const LaunchArgs& a) { return launch_mask_d<_Float16, 128>(a); }

}  // namespace attn_detail
