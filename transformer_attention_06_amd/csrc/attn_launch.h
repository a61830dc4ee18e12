// attn_launch.h — internal interface between the validated C ABI and the
// kernel launcher (not part of the public ABI).
#pragma once

#include <cstdint>

namespace attn_detail {

// Query rows owned by one workgroup (4 wavefronts x 32 rows).
constexpr int kBlockM = 128;

struct LaunchArgs {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    float* lse;
    const int32_t* pad_lens;
    int32_t dtype;
    int64_t B, S, Hq, Hkv, D;
    int causal;
    int padded;
    float scale;
    void* stream;
};

// Enqueue the kernel; returns ATTN_OK or ATTN_ERR_LAUNCH / ATTN_ERR_DEVICE.
int launch(const LaunchArgs& a);

}  // namespace attn_detail
