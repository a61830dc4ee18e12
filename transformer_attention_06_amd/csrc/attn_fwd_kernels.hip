// attn_fwd_kernels.hip — dispatch of the fused attention forward (the kernel
// template is attn_fwd_kernel.h, instantiated per element type and head dim
// in attn_fwd_<type>_d<D>.hip) and the rotary embedding pass over K.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "attn_fwd.h"
#include "attn_fwd_common.h"
#include "attn_launch.h"

namespace {

// Rotary embedding of K into K_rot, both (B, S, Hkv, D) ([ATB-guide] §8.4,
// the K half of §4.1's fifth fusion pattern).  An HBM-bound pass: one thread
// per (row, 16-byte chunk of a head row, group of up to 8 kv heads); the
// chunk's cos/sin are computed once and applied to every head of the group,
// whose 16-byte loads are all issued before the first store.  Each thread
// reads and writes the same chunks, so K_rot may be K itself.
struct RopeKParams {
    const void* k;
    void* k_out;
    const int32_t* pos;
    int64_t rows;  // B * S
    int S, Hkv, n_hg;
    double f[64];  // theta_i / 2pi, i < D/2
};

constexpr int kRopeHeads = 8;  // kv heads per thread

template <typename T, int D>
__global__ __launch_bounds__(256) void rope_k_kernel(RopeKParams rp) {
    constexpr int CH = 16 / int(sizeof(T));  // elements per chunk
    constexpr int NCH = D / CH;              // chunks per head row
    constexpr int NP = CH / 2;               // pairs per chunk
    __shared__ double f_s[D / 2];
    if (threadIdx.x < D / 2) f_s[threadIdx.x] = rp.f[threadIdx.x];
    __syncthreads();
    const int64_t gid = int64_t(blockIdx.x) * 256 + threadIdx.x;
    const int chunk = int(gid % NCH);
    const int64_t rest = gid / NCH;
    const int hg = int(rest % rp.n_hg);
    const int64_t row = rest / rp.n_hg;  // b * S + s
    if (row >= rp.rows) return;
    const int pos = rp.pos ? rp.pos[row] : int(row % rp.S);
    float cs[NP], sn[NP];
#pragma unroll
    for (int j = 0; j < NP; ++j) rope_cs<T>(pos, f_s[chunk * NP + j], cs[j], sn[j]);
    const int h0 = hg * kRopeHeads;
    const int nh = rp.Hkv - h0 < kRopeHeads ? rp.Hkv - h0 : kRopeHeads;
    const int64_t base = (row * rp.Hkv + h0) * D + int64_t(chunk) * CH;
    const u32x4* src = reinterpret_cast<const u32x4*>(static_cast<const T*>(rp.k) + base);
    u32x4* dst = reinterpret_cast<u32x4*>(static_cast<T*>(rp.k_out) + base);
    constexpr int STEP = D / CH;  // u32x4 per head row
    u32x4 v[kRopeHeads];
#pragma unroll
    for (int h = 0; h < kRopeHeads; ++h)
        if (h < nh) v[h] = src[h * STEP];
#pragma unroll
    for (int h = 0; h < kRopeHeads; ++h) {
        if (h < nh) {
            T x[CH];
            __builtin_memcpy(x, &v[h], 16);
#pragma unroll
            for (int j = 0; j < NP; ++j) {
                const float x0 = float(x[2 * j]), x1 = float(x[2 * j + 1]);
                x[2 * j] = to_t<T>(x0 * cs[j] - x1 * sn[j]);
                x[2 * j + 1] = to_t<T>(x1 * cs[j] + x0 * sn[j]);
            }
            u32x4 o;
            __builtin_memcpy(&o, x, 16);
            dst[h * STEP] = o;
        }
    }
}

template <typename T, int D>
int launch_rope_t(const attn_detail::LaunchArgs& a, void* k_out) {
    RopeKParams rp;
    rp.k = a.k;
    rp.k_out = k_out;
    rp.pos = a.rope_pos;
    rp.rows = a.B * a.S;
    rp.S = int(a.S);
    rp.Hkv = int(a.Hkv);
    rp.n_hg = int((a.Hkv + kRopeHeads - 1) / kRopeHeads);
    for (int i = 0; i < 64; ++i) rp.f[i] = i < D / 2 ? a.rope_f[i] : 0.0;
    constexpr int NCH = D / (16 / int(sizeof(T)));
    const int64_t threads = rp.rows * rp.n_hg * NCH;
    const int64_t blocks = (threads + 255) / 256;
    attn_detail::log_launch("rope_k_kernel<%s, D=%d> grid=%lld block=256 rows=%lld Hkv=%d in_place=%d",
                            attn_detail::dtype_name(a.dtype), D, (long long)blocks, (long long)rp.rows, rp.Hkv,
                            k_out == a.k ? 1 : 0);
    hipLaunchKernelGGL((rope_k_kernel<T, D>), dim3(unsigned(blocks)), dim3(256), 0,
                       static_cast<hipStream_t>(a.stream), rp);
    const hipError_t e = hipGetLastError();
    if (e == hipSuccess) return ATTN_OK;
    if (e == hipErrorNoBinaryForGpu || e == hipErrorInvalidDeviceFunction) return ATTN_ERR_DEVICE;
    return ATTN_ERR_LAUNCH;
}

template <typename T>
int launch_rope_dtype(const attn_detail::LaunchArgs& a, void* k_out) {
    return a.D == 64 ? launch_rope_t<T, 64>(a, k_out) : launch_rope_t<T, 128>(a, k_out);
}

}  // namespace

namespace attn_detail {

int launch_rope_k(const LaunchArgs& a, void* k_out) {
    switch (a.dtype) {
        case ATTN_BF16: return launch_rope_dtype<__bf16>(a, k_out);
        case ATTN_F16: return launch_rope_dtype<_Float16>(a, k_out);
        default: return launch_rope_dtype<float>(a, k_out);
    }
}

int launch_masked_tuned(const LaunchArgs& a) {
    const bool d64 = a.D == 64;
    if (a.dtype == ATTN_BF16) return d64 ? launch_fwd_mask_bf16_d64(a) : launch_fwd_mask_bf16_d128(a);
    return d64 ? launch_fwd_mask_f16_d64(a) : launch_fwd_mask_f16_d128(a);
}

int launch(const LaunchArgs& a) {
    const bool bf = a.dtype == ATTN_BF16;
    switch (a.D) {
        case 64:
            return bf ? launch_fwd_bf16_d64(a) : a.dtype == ATTN_F16 ? launch_fwd_f16_d64(a) : launch_fwd_f32_d64(a);
        case 80: return bf ? launch_fwd_bf16_d80(a) : launch_fwd_f16_d80(a);
        case 96: return bf ? launch_fwd_bf16_d96(a) : launch_fwd_f16_d96(a);
        case 112: return bf ? launch_fwd_bf16_d112(a) : launch_fwd_f16_d112(a);
        case 144: return bf ? launch_fwd_bf16_d144(a) : launch_fwd_f16_d144(a);
        case 160: return bf ? launch_fwd_bf16_d160(a) : launch_fwd_f16_d160(a);
        case 192: return bf ? launch_fwd_bf16_d192(a) : launch_fwd_f16_d192(a);
        case 256: return bf ? launch_fwd_bf16_d256(a) : launch_fwd_f16_d256(a);
        default:
            return bf ? launch_fwd_bf16_d128(a) : a.dtype == ATTN_F16 ? launch_fwd_f16_d128(a) : launch_fwd_f32_d128(a);
    }
}

}  // namespace attn_detail
