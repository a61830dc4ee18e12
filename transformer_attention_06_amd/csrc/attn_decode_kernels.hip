// attn_decode_kernels.hip — decode attention over a KV cache (gfx950).
//
// A decode step attends Sq new query rows per sequence to the L_b cached keys
// and values of that sequence, under the causal rule aligned to the end of
// the cache (row i sees key j <= L_b - Sq + i).  The serving scenario of the
// pages: the ATB introduction (hwcomputing.csdn.net/6a15a709662f9a54cb774da1)
// builds its graph operator from a causal FlashAttention with KV-cache
// management on; "CANN-ops-transformer和ATB-昇腾NPU上算子和加速库怎么配合" has
// ATB pass the cache into and out of FlashAttention every step.  With one or
// a few query rows per sequence the work is bound by reading the cache
// ("ops-transformer：Transformer算子融合与推理加速实战" §5.1: find the bound
// from bytes and FLOPs first), so the design goal is to read every cached
// byte once, coalesced, from as many workgroups as the chip has:
//
//   * one workgroup per (key chunk of 256, batch, kv head, group of 8 query
//     rows): all query heads sharing the kv head are rows of the same
//     workgroup, so K and V are read once per chunk;
//   * 16-byte loads with the head dimension across lanes (LPK lanes per key,
//     64/LPK keys per wavefront instruction): whole cache rows per load;
//   * dot products reduced over a key's lanes with DPP and lane swaps, an
//     online softmax per row in fp32 (lazily rescaled, as in the prefill
//     kernel), P·V accumulated per lane;
//   * the chunk's unnormalised (O, max, sum) goes to a caller workspace and a
//     second kernel merges the chunks by their log-sum-exp (O = Σ_s w_s O_s /
//     Σ_s w_s l_s with w_s = 2^(m_s - M)), writing O and LSE.
// This is VALU work on purpose: at one query row per key the contraction is
// far below the MFMA ridge, and the kernel is bound by HBM.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "attn_fwd.h"
#include "attn_launch.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kDecThreads = 256;  // 4 wavefronts
constexpr int kDecChunk = 256;    // keys per workgroup (64 per wavefront)
constexpr int kDecRows = 8;       // query rows per workgroup
constexpr float kDecRescale = 8.0f;

struct DecParams {
    const void* q;
    const void* k;
    const void* v;
    const int32_t* lens;
    float* ws_o;  // [n_split][B][Hq][Sq][D] unnormalised partial outputs
    float* ws_m;  // [n_split][B][Hq][Sq] partial maxima (log2 units)
    float* ws_l;  // [n_split][B][Hq][Sq] partial sums
    int B, Sq, Sk, Hq, Hkv, G, R, n_split;
    float sl2;  // scale * log2(e)
    int causal;
};

template <typename T>
__device__ __forceinline__ float to_f(T x) {
    return float(x);
}
template <typename T>
__device__ __forceinline__ T from_f(float x) {
    return static_cast<T>(x);
}

// 16 bytes of T as floats
template <typename T, int CH>
__device__ __forceinline__ void unpack(const u32x4& w, float (&x)[CH]) {
    T e[CH];
    __builtin_memcpy(e, &w, 16);
#pragma unroll
    for (int i = 0; i < CH; ++i) x[i] = to_f<T>(e[i]);
}

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, true));
}
// value of the lane 16 (or 32) lanes away
__device__ __forceinline__ float xor16(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float((threadIdx.x & 16) ? r[0] : r[1]);
}
__device__ __forceinline__ float xor32(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float((threadIdx.x & 32) ? r[0] : r[1]);
}

// Sum over the N lanes of an aligned group (N = 2..64), result in every lane
// of the group.  Steps 1 and 2 swap within quads, 4 takes the mirrored
// quad of the half-row, 8 the mirrored half of the row; after each step the
// value is uniform over the group so far, which makes the mirrors exact.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
    if constexpr (N >= 2) x += dpp<0xB1>(x);   // quad_perm [1,0,3,2]
    if constexpr (N >= 4) x += dpp<0x4E>(x);   // quad_perm [2,3,0,1]
    if constexpr (N >= 8) x += dpp<0x141>(x);  // row_half_mirror
    if constexpr (N >= 16) x += dpp<0x140>(x); // row_mirror
    if constexpr (N >= 32) x += xor16(x);
    if constexpr (N >= 64) x += xor32(x);
    return x;
}
// Max over the keys of a wavefront instruction: lanes L, L + LPK, ... (the
// value is uniform within each key's LPK lanes).
template <int LPK>
__device__ __forceinline__ float across_keys_max(float x) {
    if constexpr (LPK <= 4) x = fmaxf(x, dpp<0x141>(x));
    if constexpr (LPK <= 8) x = fmaxf(x, dpp<0x140>(x));
    if constexpr (LPK <= 16) x = fmaxf(x, xor16(x));
    if constexpr (LPK <= 32) x = fmaxf(x, xor32(x));
    return x;
}
// Sum over lanes holding the same dimensions of different keys: lane L and
// L xor (LPK << k).  Rotating a 16-lane row by 8 is the exact xor-8 partner.
template <int LPK>
__device__ __forceinline__ float across_keys_sum(float x) {
    if constexpr (LPK <= 8) x += dpp<0x128>(x);  // row_ror:8
    if constexpr (LPK <= 16) x += xor16(x);
    if constexpr (LPK <= 32) x += xor32(x);
    return x;
}

template <typename T, int D>
__global__ __launch_bounds__(kDecThreads) void decode_split_kernel(DecParams p) {
    constexpr int CH = 16 / int(sizeof(T));  // elements per lane (one 16-byte load)
    constexpr int LPK = D / CH;              // lanes per key
    constexpr int KPI = 64 / LPK;            // keys per wavefront instruction
    constexpr int NIT = kDecChunk / 4 / KPI; // instructions per wavefront
    static_assert(LPK >= 4 && LPK <= 32, "lanes per key");
    __shared__ float s_o[4][kDecRows][D];
    __shared__ float s_ml[4][kDecRows][2];

    const int split = blockIdx.x;
    const int bg = blockIdx.y;  // b * Hkv + g
    const int rg = blockIdx.z;  // group of kDecRows query rows
    const int b = bg / p.Hkv, g = bg % p.Hkv;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int c = lane % LPK;   // which 16 bytes of the row
    const int ks = lane / LPK;  // which key of the instruction
    int L = p.lens ? p.lens[b] : p.Sk;
    L = L < 0 ? 0 : (L > p.Sk ? p.Sk : L);
    const int c0 = split * kDecChunk;

    // this workgroup's rows: query head g*G + r / Sq, token r % Sq
    int hq[kDecRows], tok[kDecRows];
    bool live[kDecRows];
#pragma unroll
    for (int r = 0; r < kDecRows; ++r) {
        const int rr = rg * kDecRows + r;
        live[r] = rr < p.R;
        hq[r] = g * p.G + (live[r] ? rr / p.Sq : 0);
        tok[r] = live[r] ? rr % p.Sq : 0;
    }

    float m_run[kDecRows], l_part[kDecRows], o[kDecRows][CH];
#pragma unroll
    for (int r = 0; r < kDecRows; ++r) {
        m_run[r] = -INFINITY;
        l_part[r] = 0.0f;
#pragma unroll
        for (int e = 0; e < CH; ++e) o[r][e] = 0.0f;
    }

    if (c0 < L) {
        // Q: this lane's 16 bytes of every row, as floats
        float qf[kDecRows][CH];
#pragma unroll
        for (int r = 0; r < kDecRows; ++r) {
            if (live[r]) {
                const T* qr = static_cast<const T*>(p.q) +
                              ((int64_t(b) * p.Sq + tok[r]) * p.Hq + hq[r]) * D + c * CH;
                unpack<T, CH>(*reinterpret_cast<const u32x4*>(qr), qf[r]);
            } else {
#pragma unroll
                for (int e = 0; e < CH; ++e) qf[r][e] = 0.0f;
            }
        }
        // last key each row may see (end-aligned causal rule), exclusive
        int jend[kDecRows];
#pragma unroll
        for (int r = 0; r < kDecRows; ++r) {
            const int lim = p.causal ? L - p.Sq + tok[r] + 1 : L;
            jend[r] = live[r] ? (lim < L ? lim : L) : 0;
        }
        const int64_t kv_row = int64_t(p.Hkv) * D;  // elements between cache rows
        const T* kb = static_cast<const T*>(p.k) + (int64_t(b) * p.Sk * p.Hkv + g) * D + c * CH;
        const T* vb = static_cast<const T*>(p.v) + (int64_t(b) * p.Sk * p.Hkv + g) * D + c * CH;
        const int wbase = c0 + wave * (kDecChunk / 4);
#pragma unroll 4
        for (int it = 0; it < NIT; ++it) {
            const int j = wbase + it * KPI + ks;
            u32x4 kw = {0, 0, 0, 0}, vw = {0, 0, 0, 0};
            if (j < L) {
                kw = *reinterpret_cast<const u32x4*>(kb + int64_t(j) * kv_row);
                vw = *reinterpret_cast<const u32x4*>(vb + int64_t(j) * kv_row);
            }
            float kf[CH], vf[CH];
            unpack<T, CH>(kw, kf);
            unpack<T, CH>(vw, vf);
            float s[kDecRows];
            bool up = false;
            float mt[kDecRows];
#pragma unroll
            for (int r = 0; r < kDecRows; ++r) {
                float acc = 0.0f;
#pragma unroll
                for (int e = 0; e < CH; ++e) acc = fmaf(qf[r][e], kf[e], acc);
                acc = group_sum<LPK>(acc) * p.sl2;
                s[r] = j < jend[r] ? acc : -INFINITY;
                mt[r] = across_keys_max<LPK>(s[r]);
                up = up || (mt[r] > m_run[r] + kDecRescale);
            }
            // raise the running maxima only when some row needs it (uniform)
            if (__builtin_amdgcn_ballot_w64(up) != 0) {
#pragma unroll
                for (int r = 0; r < kDecRows; ++r) {
                    const float m_new = fmaxf(m_run[r], mt[r]);
                    const float alpha = m_new == -INFINITY ? 1.0f : __builtin_amdgcn_exp2f(m_run[r] - m_new);
                    l_part[r] *= alpha;
#pragma unroll
                    for (int e = 0; e < CH; ++e) o[r][e] *= alpha;
                    m_run[r] = m_new;
                }
            }
#pragma unroll
            for (int r = 0; r < kDecRows; ++r) {
                const float mu = m_run[r] == -INFINITY ? 0.0f : m_run[r];
                const float pr = __builtin_amdgcn_exp2f(s[r] - mu);
                l_part[r] += pr;
#pragma unroll
                for (int e = 0; e < CH; ++e) o[r][e] = fmaf(pr, vf[e], o[r][e]);
            }
        }
        // combine the keys of this wavefront: lanes with the same c
#pragma unroll
        for (int r = 0; r < kDecRows; ++r) {
            l_part[r] = across_keys_sum<LPK>(l_part[r]);
#pragma unroll
            for (int e = 0; e < CH; ++e) o[r][e] = across_keys_sum<LPK>(o[r][e]);
        }
    }
    // combine the four wavefronts through LDS, write the chunk's partial
    if (ks == 0) {
#pragma unroll
        for (int r = 0; r < kDecRows; ++r)
#pragma unroll
            for (int e = 0; e < CH; ++e) s_o[wave][r][c * CH + e] = o[r][e];
    }
    if (lane == 0) {
#pragma unroll
        for (int r = 0; r < kDecRows; ++r) {
            s_ml[wave][r][0] = m_run[r];
            s_ml[wave][r][1] = l_part[r];
        }
    }
    __syncthreads();
    for (int idx = tid; idx < kDecRows * D; idx += kDecThreads) {
        const int r = idx / D, d = idx % D;
        const int rr = rg * kDecRows + r;  // row info recomputed: r is not a constant here
        if (rr >= p.R) continue;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < 4; ++w) M = fmaxf(M, s_ml[w][r][0]);
        float lsum = 0.0f, osum = 0.0f;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const float wt = M == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(s_ml[w][r][0] - M);
            lsum += wt * s_ml[w][r][1];
            osum += wt * s_o[w][r][d];
        }
        const int64_t pi = ((int64_t(split) * p.B + b) * p.Hq + g * p.G + rr / p.Sq) * p.Sq + rr % p.Sq;
        p.ws_o[pi * D + d] = osum;
        if (d == 0) {
            p.ws_m[pi] = M;
            p.ws_l[pi] = lsum;
        }
    }
}

// Merge of the chunks: one thread per output element.
struct MergeParams {
    const float* ws_o;
    const float* ws_m;
    const float* ws_l;
    void* out;
    float* lse;
    int64_t rows;  // B * Hq * Sq partial rows, ordered (b, hq, i)
    int B, Sq, Hq, n_split;
};

template <typename T, int D>
__global__ __launch_bounds__(256) void decode_merge_kernel(MergeParams p) {
    const int64_t idx = int64_t(blockIdx.x) * 256 + threadIdx.x;
    if (idx >= p.rows * D) return;
    const int64_t row = idx / D;  // (b * Hq + hq) * Sq + i
    const int d = int(idx % D);
    float M = -INFINITY;
    for (int s = 0; s < p.n_split; ++s) M = fmaxf(M, p.ws_m[s * p.rows + row]);
    float lsum = 0.0f, osum = 0.0f;
    if (M != -INFINITY) {
        for (int s = 0; s < p.n_split; ++s) {
            const float w = __builtin_amdgcn_exp2f(p.ws_m[s * p.rows + row] - M);
            lsum += w * p.ws_l[s * p.rows + row];
            osum += w * p.ws_o[(s * p.rows + row) * D + d];
        }
    }
    const int i = int(row % p.Sq);
    const int64_t bh = row / p.Sq;
    const int hq = int(bh % p.Hq);
    const int64_t b = bh / p.Hq;
    T* orow = static_cast<T*>(p.out) + ((b * p.Sq + i) * p.Hq + hq) * D;
    orow[d] = from_f<T>(lsum > 0.0f ? osum / lsum : 0.0f);
    if (p.lse && d == 0)
        p.lse[row] = lsum > 0.0f ? (M + __builtin_amdgcn_logf(lsum)) * 0.69314718055994530942f : -INFINITY;
}

template <typename T, int D>
int launch_decode_t(const attn_detail::DecodeArgs& a) {
    DecParams dp;
    dp.q = a.q;
    dp.k = a.k;
    dp.v = a.v;
    dp.lens = a.cache_lens;
    const int64_t rows = a.B * a.Hq * a.Sq;
    float* ws = static_cast<float*>(a.workspace);
    dp.ws_o = ws;
    dp.ws_m = ws + int64_t(a.n_split) * rows * a.D;
    dp.ws_l = dp.ws_m + int64_t(a.n_split) * rows;
    dp.B = int(a.B);
    dp.Sq = int(a.Sq);
    dp.Sk = int(a.Sk);
    dp.Hq = int(a.Hq);
    dp.Hkv = int(a.Hkv);
    dp.G = int(a.Hq / a.Hkv);
    dp.R = int(dp.G * a.Sq);
    dp.n_split = a.n_split;
    dp.sl2 = a.scale * 1.44269504088896340736f;
    dp.causal = a.causal;
    const int n_rg = (dp.R + kDecRows - 1) / kDecRows;
    hipLaunchKernelGGL((decode_split_kernel<T, D>), dim3(unsigned(a.n_split), unsigned(a.B * a.Hkv), unsigned(n_rg)),
                       dim3(kDecThreads), 0, static_cast<hipStream_t>(a.stream), dp);
    hipError_t e = hipGetLastError();
    if (e == hipSuccess) {
        MergeParams mp;
        mp.ws_o = dp.ws_o;
        mp.ws_m = dp.ws_m;
        mp.ws_l = dp.ws_l;
        mp.out = a.o;
        mp.lse = a.lse;
        mp.rows = rows;
        mp.B = dp.B;
        mp.Sq = dp.Sq;
        mp.Hq = dp.Hq;
        mp.n_split = dp.n_split;
        const int64_t blocks = (rows * a.D + 255) / 256;
        hipLaunchKernelGGL((decode_merge_kernel<T, D>), dim3(unsigned(blocks)), dim3(256), 0,
                           static_cast<hipStream_t>(a.stream), mp);
        e = hipGetLastError();
    }
    if (e == hipSuccess) return ATTN_OK;
    if (e == hipErrorNoBinaryForGpu || e == hipErrorInvalidDeviceFunction) return ATTN_ERR_DEVICE;
    return ATTN_ERR_LAUNCH;
}

template <typename T>
int launch_decode_dtype(const attn_detail::DecodeArgs& a) {
    return a.D == 64 ? launch_decode_t<T, 64>(a) : launch_decode_t<T, 128>(a);
}

}  // namespace

namespace attn_detail {

int decode_splits(int64_t Sk) { return Sk > kDecChunk ? int((Sk + kDecChunk - 1) / kDecChunk) : 1; }

int launch_decode(const DecodeArgs& a) {
    switch (a.dtype) {
        case ATTN_BF16: return launch_decode_dtype<__bf16>(a);
        case ATTN_F16: return launch_decode_dtype<_Float16>(a);
        default: return launch_decode_dtype<float>(a);
    }
}

}  // namespace attn_detail
