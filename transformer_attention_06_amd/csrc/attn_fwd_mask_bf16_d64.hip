// attn_fwd_mask_bf16_d64.hip — the __bf16, D = 64 instances of the fused
// attention forward kernel (attn_fwd_kernel.h) with a mask tensor.
#include "attn_fwd_kernel.h"

namespace attn_detail {

int launch_fwd_mask_bf16_d64(const LaunchArgs& a) { return launch_mask_d<__bf16, 64>(a); }

}  // namespace attn_detail
