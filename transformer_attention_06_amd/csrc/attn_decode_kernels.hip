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
//   * one workgroup per (split of the cache, batch, kv head, group of query
//     rows): all query heads sharing the kv head are rows of the same
//     workgroup, so K and V are read once per split;
//   * 16-bit types: the query rows of a kv head (8 for a Llama-2-70B-style
//     8:1 GQA step) against the split's keys are a real, if short, dense
//     contraction, so both products run on 32x32x16 MFMA exactly as in the
//     prefill kernel's transposed form (Sᵀ = K·Qᵀ with one query row per
//     lane, Oᵀ += Vᵀ·Pᵀ; K rows taken in the permuted order that makes P an
//     MFMA operand without data movement, V read with the transposing LDS
//     read).  Splits are as few as fill every CU (so a workgroup spans many
//     keys) and each of its four wavefronts streams its share in 32-key
//     chunks through two LDS buffers of its own, loaded straight from global
//     memory, the next chunk in flight while one is computed; the wavefronts
//     combine through LDS.  Up to 32 query rows per workgroup;
//   * fp32 (a parity path): VALU dot products with the head dimension across
//     lanes, reduced with DPP and lane swaps, 256-key chunks, 8 query rows
//     per workgroup;
//   * with more than one split, each split's unnormalised (O, max, sum of the
//     rounded probabilities, exact sum) goes to a caller workspace and the
//     splits are merged by their log-sum-exp (O = Σ_s w_s O_s / Σ_s w_s l_s
//     with w_s = 2^(m_s - M)), writing O and LSE (from the exact sums): for
//     16-bit types with up to 8 splits by the workgroup of each row group
//     that finishes last (an arrival counter in the workspace, returned to
//     zero by that workgroup), otherwise by a second kernel; a single split
//     writes O and LSE itself.
// The kernel is bound by reading the cache: the MFMAs take a few per cent of
// the time the cache bytes take at full HBM bandwidth.
#include <hip/hip_runtime.h>

#include <atomic>

#include <cmath>
#include <cstdint>

#include "attn_fwd.h"
#include "attn_launch.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kDecThreads = 256;  // 4 wavefronts (fp32 kernel)
constexpr int kDecChunk = 256;    // keys per workgroup of the fp32 kernel; workspace splits per 256 keys
constexpr int kDecRows = 8;       // query rows per workgroup (fp32 kernel)
constexpr int kDecRowsMfma = 32;  // query rows per workgroup (MFMA kernel, 16-bit types)
constexpr float kDecRescale = 8.0f;

struct DecParams {
    const void* q;
    const void* k;
    const void* v;
    const int32_t* lens;
    float* ws_o;  // [n_split][B][Hq][Sq][D] unnormalised partial outputs
    float* ws_m;  // [n_split][B][Hq][Sq] partial maxima (log2 units)
    float* ws_l;  // [n_split][B][Hq][Sq] partial sums of the rounded probabilities
    float* ws_e;  // [n_split][B][Hq][Sq] partial sums of the exact probabilities (LSE)
    int B, Sq, Sk, Hq, Hkv, G, R, n_split;
    float sl2;  // scale * log2(e)
    int causal;
    int split_keys;  // streamed kernel: keys per split (a multiple of 128)
    void* o;         // streamed kernel: the output (B, Sq, Hq, D)
    float* lse;      // and the LSE (B, Hq, Sq) or null
    int* ctr;        // streamed kernel with more than one split: arrival counters,
                     // one per (batch, kv head, row group), zero on entry and exit
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
            p.ws_e[pi] = lsum;  // fp32 probabilities are not rounded
        }
    }
}

// ---- 16-bit types: both products on MFMA -----------------------------------
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

template <typename T>
struct MfmaOp;
template <>
struct MfmaOp<__bf16> {
    using op_t = bf16x8;
    static __device__ __forceinline__ f32x16 mma(op_t a, op_t b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
};
template <>
struct MfmaOp<_Float16> {
    using op_t = f16x8;
    static __device__ __forceinline__ f32x16 mma(op_t a, op_t b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    }
};

// A-operand row permutation: swap bits 2 and 3 of a 0..31 row index.  With K
// rows (and Vᵀ rows) taken in this order, accumulator register f of a lane
// in half g holds key (or head dim) 16·((f >> 3) & 1) + 8·g + (f & 7) of its
// 32-block: eight consecutive positions per register group, which are the
// eight keys the lane supplies as the P operand of the next product (and
// eight consecutive head dims of the output).
__device__ __forceinline__ int perm_row(int r) { return (r & 0x13) | ((r & 4) << 1) | ((r & 8) >> 1); }
__device__ __forceinline__ int acc_pos(int f, int g) { return 16 * ((f >> 3) & 1) + 8 * g + (f & 7); }

// Transposing LDS read: in each 16-lane group, lane 4j+q names an 8-byte
// piece (4 elements of one row); lane 4q+c receives element c of the pieces
// named by lanes 4j+q, j = 0..3.
__device__ __forceinline__ s16x4 lds_read_tr16(const void* ptr) {
    typedef s16x4 __attribute__((address_space(3))) * lds_ptr;
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_ptr)(ptr));
}

// ---- 16-bit types, streamed ---------------------------------------------------
// One workgroup per (split of the cache, batch, kv head, 32 query rows), as
// above, but a split spans many keys and each wavefront streams its share in
// 32-key chunks through two LDS buffers of its own: K and V rows go straight
// from global memory to LDS (direct loads, no registers), the loads of chunk
// c + 1 are in flight while chunk c is computed, and the loads of chunk c + 2
// are issued as soon as chunk c's operands have been read.  Nothing is shared
// between the wavefronts until the final combine, so the loop has no
// barrier.  Per chunk: Sᵀ = K·Qᵀ (one 32-key block, D/16 MFMAs), the online
// softmax (running max raised only past 2^8, as in the prefill kernel), P
// packed from the score registers, Oᵀ += Vᵀ·Pᵀ (2·D/32 MFMAs).  With one
// split the workgroup writes O and LSE itself; with up to kFoldSplits, the
// last split of a row group to finish merges them (merge_group): one launch
// either way.  More splits leave their partials to the merge kernel.
constexpr int kStrKeys = 32;   // keys per chunk
constexpr int kStrWaves = 4;

// XOR swizzle of the 16-byte slots of a K/V row (as in the prefill kernel's
// tiles): conflict-free row writes, permuted-row operand reads and
// transposing reads.
template <int NS>
__device__ __forceinline__ int str_swz(int row) {
    if constexpr (NS >= 16)
        return ((row & 3) << 2) | ((row >> 2) & 3);
    else
        return (((row >> 1) & 1) << 2) | ((row >> 2) & 3);
}

typedef int i32x4 __attribute__((ext_vector_type(4)));

// One 16-byte global load per lane into LDS at lds_byte + 16·lane
// (buffer_load_dwordx4 with LDS destination; M0 holds the LDS address).
// Assembly: the compiler does not track these writes, so every read of a
// loaded chunk is ordered by an explicit vmcnt wait of the loading wavefront
// (each wavefront reads only what it loaded itself).
__device__ __forceinline__ void str_dma16(const i32x4& rs, uint32_t lds_byte, uint32_t voff) {
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :
                 : "s"(lds_byte), "v"(voff), "s"(rs)
                 : "memory");
}

// s_waitcnt vmcnt(n) for the two counts the stream uses
__device__ __forceinline__ void str_wait(bool next_in_flight, int nld2) {
    if (next_in_flight) {
        if (nld2 == 16)
            asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
        else
            asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
    } else {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
}

// Device-scope (relaxed) atomic store and load of one float: coherent across
// the XCDs' L2 caches without cache maintenance.
__device__ __forceinline__ void coherent_store(float* p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float coherent_load(const float* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

typedef float f32x4 __attribute__((ext_vector_type(4)));
constexpr int kCoherent = 16;  // buffer cache policy: device-scope coherent (sc1)
// Launches of up to this many splits merge inside the split kernel (one
// round of loads covers them all); more splits are merged by a second
// kernel, which measured faster there (16 splits: 11.3 against 12.2 µs per
// Llama-2-70B-shaped call at B = 2, while 4 splits at B = 8 took 26.2 µs
// folded against 28.5 µs with the second kernel).
constexpr int kFoldSplits = 8;

// Buffer resource over a partial-output array of n floats (under 2^31 bytes:
// a launch with more than one split has fewer than 8192 rows and at most 256
// splits).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t partial_rsrc(const float* base, int64_t n) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(base), short(0), int(n * 4), 0x00020000);
}

// Merge of the splits of one (batch, kv head, group of 32 query rows) by the
// workgroup that arrived last: D/4 threads per row, four head dims each,
// NB splits' partials loaded at a time (device-coherent loads of the
// group's consecutive partial rows; every load of a batch is in flight at
// once, so a merge of up to NB splits waits for memory once).  O = Σ_s w_s
// O_s / Σ_s w_s l_s and LSE from Σ_s w_s e_s, with w_s = 2^(m_s - M) and M
// the largest m_s (raised batch by batch, rescaling what has been summed).
template <typename T, int D, int NB>
__device__ __forceinline__ void merge_group(const DecParams& p, __amdgpu_buffer_rsrc_t o_rs, int b, int g, int rg,
                                            int n_live, int64_t rows, int64_t grow0) {
    constexpr int TPR = D / 4;                 // threads per row
    constexpr int RPI = kStrWaves * 64 / TPR;  // rows per pass
    const int c4 = threadIdx.x % TPR;
    const int ns = p.n_split;
    for (int r = threadIdx.x / TPR; r < n_live; r += RPI) {
        const int64_t row = grow0 + r;
        float M = -INFINITY, den = 0.0f, dex = 0.0f;
        f32x4 acc = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        for (int s0 = 0; s0 < ns; s0 += NB) {
            float ms[NB], ls[NB], es[NB];
            f32x4 o[NB];
#pragma unroll
            for (int u = 0; u < NB; ++u) {
                const int s = s0 + u < ns ? s0 + u : s0;  // past the last split: re-read a valid one, weight 0
                const int64_t pi = int64_t(s) * rows + row;
                ms[u] = coherent_load(p.ws_m + pi);
                ls[u] = coherent_load(p.ws_l + pi);
                es[u] = coherent_load(p.ws_e + pi);
                o[u] = __builtin_bit_cast(
                    f32x4, __builtin_amdgcn_raw_buffer_load_b128(o_rs, int(uint32_t(pi * D * 4) + uint32_t(c4) * 16u),
                                                                 0, kCoherent));
            }
            float bm = M;
#pragma unroll
            for (int u = 0; u < NB; ++u) {
                if (s0 + u >= ns) ms[u] = -INFINITY;
                bm = fmaxf(bm, ms[u]);
            }
            if (bm == -INFINITY) continue;  // no visible key in any split so far
            const float a = M == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(M - bm);
            den *= a;
            dex *= a;
            acc *= a;
            M = bm;
#pragma unroll
            for (int u = 0; u < NB; ++u) {
                const float w = ms[u] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(ms[u] - M);
                den += w * ls[u];
                dex += w * es[u];
                acc += w * o[u];
            }
        }
        const float inv = den > 0.0f ? 1.0f / den : 0.0f;
        const int rr = rg * kDecRowsMfma + r;
        const int hq = g * p.G + rr / p.Sq, tok = rr % p.Sq;
        T o4[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) o4[i] = from_f<T>(acc[i] * inv);
        T* orow = static_cast<T*>(p.o) + ((int64_t(b) * p.Sq + tok) * p.Hq + hq) * D + c4 * 4;
        *reinterpret_cast<uint64_t*>(orow) = __builtin_bit_cast(uint64_t, o4);
        if (c4 == 0 && p.lse)
            p.lse[row] = dex > 0.0f ? (M + __builtin_amdgcn_logf(dex)) * 0.69314718055994530942f : -INFINITY;
    }
}

template <typename T, int D>
__global__ __launch_bounds__(kStrWaves * 64, 1) void decode_stream_kernel(DecParams p) {
    using op_t = typename MfmaOp<T>::op_t;
    constexpr int CH = 8;                       // elements per 16-byte slot
    constexpr int NS = D / CH;                  // slots per row
    constexpr int ROW_B = D * 2;                // bytes per row
    constexpr int TILE_E = kStrKeys * D;        // elements per K (or V) chunk
    constexpr int NLD = kStrKeys * ROW_B / 1024;  // 1 KiB loads per chunk tile
    constexpr int RPL = 1024 / ROW_B;           // rows per load
    constexpr int NC = D / 16;                  // Sᵀ MFMAs per chunk
    constexpr int NDB = D / 32;                 // 32-dim blocks of O
    static_assert(NLD * 1024 == kStrKeys * ROW_B && 2 * NLD <= 16, "chunk loads");
    // per wavefront: buffers 0 and 1, each a K tile then a V tile
    __shared__ __attribute__((aligned(1024))) T lds[kStrWaves * 2 * 2 * TILE_E];
    __shared__ float s_ml[kStrWaves][3][64];
    static_assert(kStrWaves * NDB * 16 * 64 * 4 <= int(sizeof(lds)), "combine stash fits the tiles");

    const int split = blockIdx.x;
    const int bg = blockIdx.y;  // b * Hkv + g
    const int rg = blockIdx.z;  // group of 32 query rows
    const int b = bg / p.Hkv, g = bg % p.Hkv;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x >> 6));
    const int r = lane & 31, gl = lane >> 5;
    int L = p.lens ? p.lens[b] : p.Sk;
    L = L < 0 ? 0 : (L > p.Sk ? p.Sk : L);

    const int rr = rg * kDecRowsMfma + r;
    const bool live = rr < p.R;
    const int hq = g * p.G + (live ? rr / p.Sq : 0);
    const int tok = live ? rr % p.Sq : 0;
    int jend = 0;  // keys j < jend are visible to this row
    if (live) {
        jend = p.causal ? L - p.Sq + tok + 1 : L;
        jend = jend < 0 ? 0 : (jend > L ? L : jend);
    }

    // this wavefront's keys: [w0, w1), in chunks of 32
    const int per_wave = p.split_keys / kStrWaves;
    const int w0 = split * p.split_keys + wave * per_wave;
    int w1 = w0 + per_wave;
    w1 = w1 < L ? w1 : L;
    const int n_ch = w1 > w0 ? (w1 - w0 + kStrKeys - 1) / kStrKeys : 0;

    // Q operand of the lane's row: head dims 16c + 8gl .. +7 (rows past the
    // group read the group's first row; their results are never written);
    // loaded before any chunk so that its wait covers nothing else
    op_t qop[NC];
    const T* qr = static_cast<const T*>(p.q) + ((int64_t(b) * p.Sq + tok) * p.Hq + hq) * D + 8 * gl;
#pragma unroll
    for (int c = 0; c < NC; ++c) qop[c] = *reinterpret_cast<const op_t*>(qr + 16 * c);
#pragma unroll
    for (int c = 0; c < NC; ++c) asm volatile("" : "+v"(qop[c]));

    // loads: rows k0 + [0, 32) of this (batch, kv head) slice, through a
    // resource ending after row L - 1 (rows at or past L read as zero)
    const uint32_t row_stride = uint32_t(p.Hkv) * uint32_t(ROW_B);
    const T* kbase = static_cast<const T*>(p.k) + (int64_t(b) * p.Sk * p.Hkv + g) * D;
    const T* vbase = static_cast<const T*>(p.v) + (int64_t(b) * p.Sk * p.Hkv + g) * D;
    const int lr = lane / (ROW_B / 16), ps = lane % (ROW_B / 16);
    uint32_t voff[NLD];
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
        const int row = i * RPL + lr;
        voff[i] = uint32_t(row) * row_stride + uint32_t((ps ^ str_swz<NS>(row)) * 16);
    }
    const uint32_t lds_w = __builtin_amdgcn_readfirstlane(
        uint32_t(reinterpret_cast<uintptr_t>(lds)) + uint32_t(wave * 2 * 2 * TILE_E * 2));
    auto issue = [&](int c) __attribute__((always_inline)) {
        const int k0 = w0 + c * kStrKeys;
        const int valid = L - k0 < kStrKeys ? L - k0 : kStrKeys;  // >= 1: k0 < L
        const uint32_t rec = uint32_t(valid - 1) * row_stride + uint32_t(ROW_B);
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const uint64_t a = reinterpret_cast<uint64_t>(t == 0 ? kbase : vbase) + uint64_t(k0) * row_stride;
            const i32x4 rs{__builtin_amdgcn_readfirstlane(int(uint32_t(a))),
                           __builtin_amdgcn_readfirstlane(int(uint32_t(a >> 32) & 0xffff)),
                           __builtin_amdgcn_readfirstlane(int(rec)), 0x00020000};
            const uint32_t dst = lds_w + uint32_t((((c & 1) * 2 + t) * TILE_E) * 2);
#pragma unroll
            for (int i = 0; i < NLD; ++i) str_dma16(rs, dst + uint32_t(i * 1024), voff[i]);
        }
    };

    // per-lane LDS read offsets (elements within a tile)
    const int prow = perm_row(r);
    const int xk = str_swz<NS>(prow);
    const int tr_key = (r & 15) >> 2;
    const int tr_col = 16 * (r >> 4) + 4 * (((r & 1) << 1) | ((r >> 1) & 1));
    int v_off[NDB][2];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int key = 8 * gl + 4 * h + tr_key;
            const int col = 32 * db + tr_col;
            v_off[db][h] = key * D + (((col / CH) ^ str_swz<NS>(key)) * CH) + col % CH;
        }
    const T* lds_wave = lds + wave * 2 * 2 * TILE_E;

    f32x16 oacc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) oacc[db] = f32x16{};
    float m_run = -INFINITY, l_run = 0.0f, e_run = 0.0f;

    if (n_ch > 0) issue(0);
    if (n_ch > 1) issue(1);
    for (int c = 0; c < n_ch; ++c) {
        str_wait(c + 1 < n_ch, 2 * NLD);  // chunk c landed (chunk c + 1 may still be in flight)
        const T* kt = lds_wave + (c & 1) * 2 * TILE_E;
        const T* vt = kt + TILE_E;
        const int k0 = w0 + c * kStrKeys;
        // Sᵀ: virtual row r of the block is key k0 + perm_row(r)
        f32x16 sacc = f32x16{};
#pragma unroll
        for (int cc = 0; cc < NC; ++cc) {
            const op_t ka = *reinterpret_cast<const op_t*>(kt + prow * D + (((2 * cc + gl) ^ xk) * CH));
            sacc = MfmaOp<T>::mma(ka, qop[cc], sacc);
        }
        // scores in log2 units, hidden keys -inf; this chunk's row max
        float mx = -INFINITY;
#pragma unroll
        for (int f = 0; f < 16; ++f) {
            const int key = k0 + acc_pos(f, gl);
            const float sv = key < jend ? sacc[f] * p.sl2 : -INFINITY;
            sacc[f] = sv;
            mx = fmaxf(mx, sv);
        }
        mx = fmaxf(mx, xor32(mx));
        // raise the running max only when some row of the wavefront gains
        // more than 2^8 (the exponentials then stay below 2^8)
        const bool resc = __builtin_amdgcn_ballot_w64(mx > m_run + kDecRescale) != 0;
        if (resc) {
            const float m_new = fmaxf(m_run, mx);
            const float alpha = m_new == -INFINITY ? 1.0f : __builtin_amdgcn_exp2f(m_run - m_new);
            l_run *= alpha;
            e_run *= alpha;
#pragma unroll
            for (int db = 0; db < NDB; ++db) oacc[db] *= alpha;
            m_run = m_new;
        }
        const float mu = m_run == -INFINITY ? 0.0f : m_run;
        op_t pop[2];  // P operand of 16-key step kc: registers 8kc .. 8kc+7
#pragma unroll
        for (int kc = 0; kc < 2; ++kc)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float pe = __builtin_amdgcn_exp2f(sacc[8 * kc + e] - mu);
                const T pr = static_cast<T>(pe);
                e_run += pe;
                l_run += float(pr);
                pop[kc][e] = pr;
            }
        // Oᵀ += Vᵀ·Pᵀ
#pragma unroll
        for (int kc = 0; kc < 2; ++kc)
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
                s16x4 half[2];
#pragma unroll
                for (int h = 0; h < 2; ++h) half[h] = lds_read_tr16(vt + 16 * kc * D + v_off[db][h]);
                const op_t va =
                    __builtin_bit_cast(op_t, __builtin_shufflevector(half[0], half[1], 0, 1, 2, 3, 4, 5, 6, 7));
                oacc[db] = MfmaOp<T>::mma(va, pop[kc], oacc[db]);
            }
        // this chunk's operands are read: its buffers take chunk c + 2
        if (c + 2 < n_ch) {
            __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
            issue(c + 2);
        }
    }
    // rows' sums over both halves of the wavefront (keys 8gl .. of each block)
    l_run += xor32(l_run);
    e_run += xor32(e_run);

    // combine the four wavefronts through LDS (every chunk's loads have
    // landed: the last wait was vmcnt(0))
    __syncthreads();
    float* stash = reinterpret_cast<float*>(lds);
    constexpr int DP = D + 4;  // padded row of the staged partial rows
    float* c_rows = stash + kStrWaves * NDB * 16 * 64;
    static_assert((kStrWaves * NDB * 16 * 64 + kDecRowsMfma * DP) * 4 <= int(sizeof(lds)), "staged rows fit");
    __shared__ float s_part[3][kDecRowsMfma];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int f = 0; f < 16; ++f) stash[((wave * NDB + db) * 16 + f) * 64 + lane] = oacc[db][f];
    s_ml[wave][0][lane] = m_run;
    s_ml[wave][1][lane] = l_run;
    s_ml[wave][2][lane] = e_run;
    __syncthreads();
    if (wave < NDB && live) {
        const int db = wave;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < kStrWaves; ++w) M = fmaxf(M, s_ml[w][0][lane]);
        float wt[kStrWaves], lt = 0.0f, et = 0.0f;
#pragma unroll
        for (int w = 0; w < kStrWaves; ++w) {
            wt[w] = M == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(s_ml[w][0][lane] - M);
            lt += wt[w] * s_ml[w][1][lane];
            et += wt[w] * s_ml[w][2][lane];
        }
        if (p.n_split == 1) {
            // the whole cache in this workgroup: O and LSE directly
            const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
            T* orow = static_cast<T*>(p.o) + ((int64_t(b) * p.Sq + tok) * p.Hq + hq) * D + 32 * db + 8 * gl;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                T o8[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int f = 8 * h + e;
                    float acc = 0.0f;
#pragma unroll
                    for (int w = 0; w < kStrWaves; ++w) acc += wt[w] * stash[((w * NDB + db) * 16 + f) * 64 + lane];
                    o8[e] = from_f<T>(acc * inv);
                }
                *reinterpret_cast<u32x4*>(orow + 16 * h) = *reinterpret_cast<const u32x4*>(o8);
            }
            if (db == 0 && gl == 0 && p.lse)
                p.lse[(int64_t(b) * p.Hq + hq) * p.Sq + tok] =
                    et > 0.0f ? (M + __builtin_amdgcn_logf(et)) * 0.69314718055994530942f : -INFINITY;
        } else if (!p.ctr) {
            // partials for the merge kernel, straight from the registers
            const int64_t pi = ((int64_t(split) * p.B + b) * p.Hq + hq) * p.Sq + tok;
            float* dst = p.ws_o + pi * D + 32 * db + 8 * gl;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                float o8[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int f = 8 * h + e;
                    float acc = 0.0f;
#pragma unroll
                    for (int w = 0; w < kStrWaves; ++w) acc += wt[w] * stash[((w * NDB + db) * 16 + f) * 64 + lane];
                    o8[e] = acc;
                }
                reinterpret_cast<u32x4*>(dst + 16 * h)[0] = *reinterpret_cast<const u32x4*>(&o8[0]);
                reinterpret_cast<u32x4*>(dst + 16 * h)[1] = *reinterpret_cast<const u32x4*>(&o8[4]);
            }
            if (db == 0 && gl == 0) {
                p.ws_m[pi] = M;
                p.ws_l[pi] = lt;
                p.ws_e[pi] = et;
            }
        } else {
            // this split's combined rows, row-major, for the coalesced
            // device-coherent stores below
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int f = 8 * h + e;
                    float acc = 0.0f;
#pragma unroll
                    for (int w = 0; w < kStrWaves; ++w) acc += wt[w] * stash[((w * NDB + db) * 16 + f) * 64 + lane];
                    c_rows[r * DP + 32 * db + 8 * gl + 16 * h + e] = acc;
                }
            if (db == 0 && gl == 0) {
                s_part[0][r] = M;
                s_part[1][r] = lt;
                s_part[2][r] = et;
            }
        }
    }
    if (p.n_split == 1 || !p.ctr) return;

    // More than one split, with arrival counters: this split's partial (O,
    // max, sums) of the group's live rows goes to the workspace, and the last
    // split of this (batch, kv head, row group) to arrive merges all of them
    // and returns the counter to zero for the next call on this workspace.
    // The group's rows are consecutive rows of the partial arrays, so the
    // stores and the merge's loads are whole 16-byte vectors, coalesced.
    // They are device-coherent accesses (sc1), served where all of the chip's
    // L2 caches agree, so no cache writeback or invalidation is needed (a
    // device-scope fence writes back and invalidates this XCD's whole L2);
    // the arrival is counted after every thread's stores have completed, and
    // the merge's loads are issued after the count.
    const int n_live = p.R - rg * kDecRowsMfma < kDecRowsMfma ? p.R - rg * kDecRowsMfma : kDecRowsMfma;
    const int64_t rows = int64_t(p.B) * p.Hq * p.Sq;
    const int64_t grow0 = (int64_t(b) * p.Hq + int64_t(g) * p.G) * p.Sq + rg * kDecRowsMfma;  // group's first row
    const __amdgpu_buffer_rsrc_t o_rs = partial_rsrc(p.ws_o, int64_t(p.n_split) * rows * D);
    __syncthreads();
    {
        const uint32_t base = uint32_t((int64_t(split) * rows + grow0) * D * 4);
        for (int i = threadIdx.x; i * 4 < n_live * D; i += kStrWaves * 64) {
            const int rw = i * 4 / D, col = i * 4 % D;
            const i32x4 v = __builtin_bit_cast(i32x4, *reinterpret_cast<const f32x4*>(c_rows + rw * DP + col));
            __builtin_amdgcn_raw_buffer_store_b128(v, o_rs, int(base + uint32_t(i) * 16u), 0, kCoherent);
        }
        if (int(threadIdx.x) < n_live) {
            const int64_t pi = int64_t(split) * rows + grow0 + threadIdx.x;
            coherent_store(p.ws_m + pi, s_part[0][threadIdx.x]);
            coherent_store(p.ws_l + pi, s_part[1][threadIdx.x]);
            coherent_store(p.ws_e + pi, s_part[2][threadIdx.x]);
        }
    }
    __shared__ int s_last;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (threadIdx.x == 0) {
        int* ctr = p.ctr + (blockIdx.y * gridDim.z + blockIdx.z);
        const int arrived = __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_last = arrived == p.n_split - 1;
        if (s_last) __hip_atomic_store(ctr, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    if (!s_last) return;
    merge_group<T, D, kFoldSplits>(p, o_rs, b, g, rg, n_live, rows, grow0);
}

// Merge kernel (the fp32 kernel's chunks, and the 16-bit kernel's splits when
// there are more than kFoldSplits): one wavefront per output row; lanes
// read the chunk maxima and sums side by side, then accumulate the weighted
// partial outputs with the head dimension across lanes, eight chunks' loads
// in flight at once.
struct MergeParams {
    const float* ws_o;
    const float* ws_m;
    const float* ws_l;
    const float* ws_e;
    void* out;
    float* lse;
    int64_t rows;  // B * Hq * Sq partial rows, ordered (b, hq, i)
    int B, Sq, Hq, n_split;
};

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
    return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
    return x;
}

template <typename T, int D>
__global__ __launch_bounds__(256) void decode_merge_kernel(MergeParams p) {
    constexpr int DPL = D / 64;  // head dims per lane
    const int lane = threadIdx.x & 63;
    const int64_t row = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);  // (b * Hq + hq) * Sq + i
    if (row >= p.rows) return;                                          // whole wavefront
    float M = -INFINITY;
    for (int s = lane; s < p.n_split; s += 64) M = fmaxf(M, p.ws_m[int64_t(s) * p.rows + row]);
    M = wave_max(M);
    float den = 0.0f, dex = 0.0f, acc[DPL];
#pragma unroll
    for (int i = 0; i < DPL; ++i) acc[i] = 0.0f;
    if (M != -INFINITY) {
        for (int s0 = 0; s0 < p.n_split; s0 += 64) {
            const int s = s0 + lane;
            float w = 0.0f;
            if (s < p.n_split) {
                const int64_t pi = int64_t(s) * p.rows + row;
                w = __builtin_amdgcn_exp2f(p.ws_m[pi] - M);
                den += w * p.ws_l[pi];
                dex += w * p.ws_e[pi];
            }
            const int ns = p.n_split - s0 < 64 ? p.n_split - s0 : 64;
            int t = 0;
            for (; t + 8 <= ns; t += 8) {
                float v[8][DPL];
#pragma unroll
                for (int u = 0; u < 8; ++u)
#pragma unroll
                    for (int i = 0; i < DPL; ++i)
                        v[u][i] = p.ws_o[(int64_t(s0 + t + u) * p.rows + row) * D + lane + 64 * i];
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const float wt = __shfl(w, t + u);
#pragma unroll
                    for (int i = 0; i < DPL; ++i) acc[i] += wt * v[u][i];
                }
            }
            for (; t < ns; ++t) {
                const float wt = __shfl(w, t);
#pragma unroll
                for (int i = 0; i < DPL; ++i)
                    acc[i] += wt * p.ws_o[(int64_t(s0 + t) * p.rows + row) * D + lane + 64 * i];
            }
        }
    }
    den = wave_sum(den);
    dex = wave_sum(dex);
    const int i_tok = int(row % p.Sq);
    const int64_t bh = row / p.Sq;
    const int hq = int(bh % p.Hq);
    const int64_t b = bh / p.Hq;
    T* orow = static_cast<T*>(p.out) + ((b * p.Sq + i_tok) * p.Hq + hq) * D;
    const float inv = den > 0.0f ? 1.0f / den : 0.0f;
#pragma unroll
    for (int i = 0; i < DPL; ++i) orow[lane + 64 * i] = from_f<T>(acc[i] * inv);
    if (p.lse && lane == 0)
        p.lse[row] = dex > 0.0f ? (M + __builtin_amdgcn_logf(dex)) * 0.69314718055994530942f : -INFINITY;
}

// Splits of the streamed kernel: enough workgroups for every CU (256), no
// more splits than the workspace was sized for (attn_decode_workspace_bytes:
// one per 256 cached keys), keys per split a multiple of 4 wavefronts x 32.
inline void stream_splits(int64_t units, int64_t Sk, int max_split, int& n_split, int& split_keys) {
    int64_t ns = (256 + units - 1) / units;
    ns = ns < 1 ? 1 : (ns > max_split ? max_split : ns);
    int64_t sk = (Sk + ns - 1) / ns;
    sk = (sk + 127) / 128 * 128;
    sk = sk < 128 ? 128 : sk;
    split_keys = int(sk);
    n_split = int(Sk > 0 ? (Sk + sk - 1) / sk : 1);
}

template <typename T, int D>
int launch_decode_t(const attn_detail::DecodeArgs& a) {
    DecParams dp;
    dp.q = a.q;
    dp.k = a.k;
    dp.v = a.v;
    dp.lens = a.cache_lens;
    const int64_t rows = a.B * a.Hq * a.Sq;
    int n_split = a.n_split;
    dp.split_keys = 0;
    if constexpr (sizeof(T) == 2) {
        const int64_t n_rg = (int64_t(a.Hq / a.Hkv) * a.Sq + kDecRowsMfma - 1) / kDecRowsMfma;
        stream_splits(a.B * a.Hkv * n_rg, a.Sk, a.n_split, n_split, dp.split_keys);
    }
    // the workspace: arrival counters, then the partial results
    dp.ctr = nullptr;
    float* ws = reinterpret_cast<float*>(static_cast<char*>(a.workspace) + attn_detail::kDecodeCounterBytes);
    dp.ws_o = ws;
    dp.ws_m = ws + int64_t(n_split) * rows * a.D;
    dp.ws_l = dp.ws_m + int64_t(n_split) * rows;
    dp.ws_e = dp.ws_l + int64_t(n_split) * rows;
    dp.o = a.o;
    dp.lse = a.lse;
    dp.B = int(a.B);
    dp.Sq = int(a.Sq);
    dp.Sk = int(a.Sk);
    dp.Hq = int(a.Hq);
    dp.Hkv = int(a.Hkv);
    dp.G = int(a.Hq / a.Hkv);
    dp.R = int(dp.G * a.Sq);
    dp.n_split = n_split;
    dp.sl2 = a.scale * 1.44269504088896340736f;
    dp.causal = a.causal;
    if constexpr (sizeof(T) == 2) {
        const int n_rg = (dp.R + kDecRowsMfma - 1) / kDecRowsMfma;
        // more than one split only when the groups number fewer than 256
        // (stream_splits), so their counters fit the workspace's header
        if (n_split > 1 && a.B * a.Hkv * n_rg * int64_t(sizeof(int)) > attn_detail::kDecodeCounterBytes)
            return ATTN_ERR_LAUNCH;
        if (n_split > 1 && n_split <= kFoldSplits) dp.ctr = static_cast<int*>(a.workspace);
        attn_detail::log_launch("decode_stream_kernel<%s, D=%d> grid=(%d, %lld, %d) block=%d split_keys=%d Sk=%lld "
                                "Sq=%lld",
                                attn_detail::dtype_name(a.dtype), D, n_split, (long long)(a.B * a.Hkv), n_rg,
                                kStrWaves * 64, dp.split_keys, (long long)a.Sk, (long long)a.Sq);
        hipLaunchKernelGGL((decode_stream_kernel<T, D>), dim3(unsigned(n_split), unsigned(a.B * a.Hkv), unsigned(n_rg)),
                           dim3(kStrWaves * 64), 0, static_cast<hipStream_t>(a.stream), dp);
    } else {
        const int n_rg = (dp.R + kDecRows - 1) / kDecRows;
        attn_detail::log_launch("decode_split_kernel<%s, D=%d> grid=(%d, %lld, %d) block=%d Sk=%lld Sq=%lld",
                                attn_detail::dtype_name(a.dtype), D, a.n_split, (long long)(a.B * a.Hkv), n_rg,
                                kDecThreads, (long long)a.Sk, (long long)a.Sq);
        hipLaunchKernelGGL((decode_split_kernel<T, D>), dim3(unsigned(a.n_split), unsigned(a.B * a.Hkv), unsigned(n_rg)),
                           dim3(kDecThreads), 0, static_cast<hipStream_t>(a.stream), dp);
    }
    hipError_t e = hipGetLastError();
    // the streamed kernel writes the output itself with one split, or with
    // up to kFoldSplits (its last split merges)
    if (e == hipSuccess && (sizeof(T) == 4 || (n_split > 1 && dp.ctr == nullptr))) {
        MergeParams mp;
        mp.ws_o = dp.ws_o;
        mp.ws_m = dp.ws_m;
        mp.ws_l = dp.ws_l;
        mp.ws_e = dp.ws_e;
        mp.out = a.o;
        mp.lse = a.lse;
        mp.rows = rows;
        mp.B = dp.B;
        mp.Sq = dp.Sq;
        mp.Hq = dp.Hq;
        mp.n_split = dp.n_split;
        const int64_t blocks = (rows + 3) / 4;
        attn_detail::log_launch("decode_merge_kernel<%s, D=%d> grid=%lld block=256 splits=%d",
                                attn_detail::dtype_name(a.dtype), D, (long long)blocks, mp.n_split);
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

// Workspace of the allocation-free entry point (attn_fwd_decode_noalloc): a
// fixed device array, one copy per GPU for the life of the process.  In host
// code the name below is a host-side stand-in, never a device address: the
// device address is looked up with hipGetSymbolAddress, once per device.
// Without an initialiser the array is zero when the code object is loaded
// (static storage), which is what its leading arrival counters need.
static __device__ __align__(256) float attn_decode_scratch[attn_detail::kDecodeScratchBytes / sizeof(float)];

namespace attn_detail {

int decode_scratch(void** ws) {
    constexpr int kMaxDevices = 64;
    static std::atomic<void*> addr[kMaxDevices];
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return ATTN_ERR_DEVICE;
    void* p = addr[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        // with this device current: its copy of the array (two threads that
        // race here store the same address)
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(attn_decode_scratch)) != hipSuccess || p == nullptr)
            return ATTN_ERR_DEVICE;
        addr[dev].store(p, std::memory_order_release);
    }
    *ws = p;
    return ATTN_OK;
}

int64_t decode_splits(int64_t Sk) { return Sk > kDecChunk ? Sk / kDecChunk + (Sk % kDecChunk != 0) : 1; }

int launch_decode(const DecodeArgs& a) {
    switch (a.dtype) {
        case ATTN_BF16: return launch_decode_dtype<__bf16>(a);
        case ATTN_F16: return launch_decode_dtype<_Float16>(a);
        default: return launch_decode_dtype<float>(a);
    }
}

}  // namespace attn_detail
