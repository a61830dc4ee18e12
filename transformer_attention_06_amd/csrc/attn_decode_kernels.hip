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
//   * one workgroup per (key chunk of 256, batch, kv head, group of query
//     rows): all query heads sharing the kv head are rows of the same
//     workgroup, so K and V are read once per chunk;
//   * 16-bit types: the query rows of a kv head (8 for a Llama-2-70B-style
//     8:1 GQA step) against the chunk's keys are a real, if short, dense
//     contraction, so both products run on 32x32x16 MFMA exactly as in the
//     prefill kernel's transposed form (Sᵀ = K·Qᵀ with one query row per
//     lane, Oᵀ += Vᵀ·Pᵀ): K and Q operands are 16-byte global loads straight
//     into registers (K rows taken in the permuted order that makes P an MFMA
//     operand without data movement), V goes through LDS and is read back
//     with the transposing LDS read.  Each wavefront owns 64 keys, computes
//     their scores, softmax and P·V in one pass, and the four wavefronts
//     combine through LDS.  Up to 32 query rows per workgroup;
//   * fp32 (a parity path): VALU dot products with the head dimension across
//     lanes, reduced with DPP and lane swaps, 8 query rows per workgroup;
//   * the chunk's unnormalised (O, max, sum of the rounded probabilities,
//     exact sum) goes to a caller workspace and a second kernel, one
//     wavefront per output row, merges the chunks by their log-sum-exp
//     (O = Σ_s w_s O_s / Σ_s w_s l_s with w_s = 2^(m_s - M)), writing O and
//     LSE (from the exact sums).
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

constexpr int kDecThreads = 256;  // 4 wavefronts
constexpr int kDecChunk = 256;    // keys per workgroup (64 per wavefront)
constexpr int kDecRows = 8;       // query rows per workgroup (fp32 kernel)
constexpr int kDecRowsMfma = 32;  // query rows per workgroup (MFMA kernel)
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

template <typename T, int D>
__global__ __launch_bounds__(kDecThreads, 2) void decode_mfma_kernel(DecParams p) {
    using op_t = typename MfmaOp<T>::op_t;
    constexpr int KW = kDecChunk / 4;  // keys per wavefront (64)
    constexpr int NC = D / 16;         // MFMA steps along D for Sᵀ
    constexpr int NDB = D / 32;        // 32-dim blocks of Oᵀ
    constexpr int ROWP = D + 8;        // LDS row pitch of the V tile (elements): rows shift by 16 bytes
    constexpr int CPR = D / 8;         // 16-byte chunks per cache row
    constexpr int NVL = KW * CPR / 64; // V chunks per lane
    static_assert(4 * NDB * 16 * 64 * 4 <= 4 * KW * ROWP * int(sizeof(T)), "combine stash fits the V tiles");
    __shared__ __attribute__((aligned(16))) T vt[4 * KW * ROWP];
    __shared__ float s_ml[4][3][64];

    const int split = blockIdx.x;
    const int bg = blockIdx.y;  // b * Hkv + g
    const int rg = blockIdx.z;  // group of 32 query rows
    const int b = bg / p.Hkv, g = bg % p.Hkv;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r = lane & 31, gl = lane >> 5;
    int L = p.lens ? p.lens[b] : p.Sk;
    L = L < 0 ? 0 : (L > p.Sk ? p.Sk : L);
    const int k0 = split * kDecChunk + wave * KW;  // this wavefront's first key

    // this lane's query row (the same for both halves of the wavefront)
    const int rr = rg * kDecRowsMfma + r;
    const bool live = rr < p.R;
    const int hq = g * p.G + (live ? rr / p.Sq : 0);
    const int tok = live ? rr % p.Sq : 0;
    int jend = 0;  // keys j < jend are visible to this row (end-aligned causal rule)
    if (live) {
        jend = p.causal ? L - p.Sq + tok + 1 : L;
        jend = jend < 0 ? 0 : (jend > L ? L : jend);
    }

    const int64_t kv_row = int64_t(p.Hkv) * D;  // elements between cache rows
    const T* kb = static_cast<const T*>(p.k) + (int64_t(b) * p.Sk * p.Hkv + g) * D;
    const T* vb = static_cast<const T*>(p.v) + (int64_t(b) * p.Sk * p.Hkv + g) * D;
    T* vw = vt + wave * KW * ROWP;

    // Loads without branches, so that every load of the wavefront is in
    // flight at once: cache rows past L are read as row L-1 (their scores
    // are hidden, so they only meet P = 0), and a wavefront whose 64 keys
    // all lie past L loads nothing (a wavefront-uniform branch).
    const bool any = k0 < L;
    const int klast = L - 1;
    // V: the wavefront's 64 cache rows into its LDS tile
    u32x4 vreg[NVL];
    // K operands: block blk, virtual row r is key k0 + 32·blk + perm_row(r);
    // the lane holds head dims 16c + 8gl .. +7
    op_t kop[2][NC];
    if (any) {
#pragma unroll
        for (int i = 0; i < NVL; ++i) {
            const int ch = lane + 64 * i, key = k0 + ch / CPR, c8 = ch % CPR;
            vreg[i] = *reinterpret_cast<const u32x4*>(vb + int64_t(key < L ? key : klast) * kv_row + 8 * c8);
        }
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) {
            const int key = k0 + 32 * blk + perm_row(r);
            const T* kr = kb + int64_t(key < L ? key : klast) * kv_row + 8 * gl;
#pragma unroll
            for (int c = 0; c < NC; ++c) kop[blk][c] = *reinterpret_cast<const op_t*>(kr + 16 * c);
        }
    } else {
#pragma unroll
        for (int i = 0; i < NVL; ++i) vreg[i] = u32x4{0, 0, 0, 0};
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
#pragma unroll
            for (int c = 0; c < NC; ++c) kop[blk][c] = op_t{};
    }
    // Q operand: the lane's row, head dims 16c + 8gl .. +7 (rows past the
    // group read the group's first row: their keys are all hidden and their
    // results are never written)
    op_t qop[NC];
    const T* qr = static_cast<const T*>(p.q) + ((int64_t(b) * p.Sq + tok) * p.Hq + hq) * D + 8 * gl;
#pragma unroll
    for (int c = 0; c < NC; ++c) qop[c] = *reinterpret_cast<const op_t*>(qr + 16 * c);

#pragma unroll
    for (int i = 0; i < NVL; ++i) {
        const int ch = lane + 64 * i;
        *reinterpret_cast<u32x4*>(vw + (ch / CPR) * ROWP + 8 * (ch % CPR)) = vreg[i];
    }

    // Sᵀ = K·Qᵀ for the 64 keys
    f32x16 sacc[2];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
        sacc[blk] = f32x16{};
#pragma unroll
        for (int c = 0; c < NC; ++c) sacc[blk] = MfmaOp<T>::mma(kop[blk][c], qop[c], sacc[blk]);
    }

    // softmax over the wavefront's keys (scores in log2 units)
    float mx = -INFINITY;
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int f = 0; f < 16; ++f) {
            const int key = k0 + 32 * blk + acc_pos(f, gl);
            const float sv = key < jend ? sacc[blk][f] * p.sl2 : -INFINITY;
            sacc[blk][f] = sv;
            mx = fmaxf(mx, sv);
        }
    mx = fmaxf(mx, xor32(mx));
    const float mu = mx == -INFINITY ? 0.0f : mx;
    float lsum = 0.0f, lex = 0.0f;
    op_t pop[2][2];  // P operand of block blk, 16-key step kc: registers 8kc .. 8kc+7
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int kc = 0; kc < 2; ++kc)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float pe = __builtin_amdgcn_exp2f(sacc[blk][8 * kc + e] - mu);
                const T pr = static_cast<T>(pe);
                lex += pe;
                lsum += float(pr);
                pop[blk][kc][e] = pr;
            }
    lsum += xor32(lsum);
    lex += xor32(lex);

    // the tile was written by this wavefront's own lanes: wait for the writes
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    __builtin_amdgcn_wave_barrier();

    // Oᵀ += Vᵀ·Pᵀ: Vᵀ rows (head dims) in the permuted order, read transposed
    const int tr_key = (r & 15) >> 2;
    const int tr_col = 16 * (r >> 4) + 4 * (((r & 1) << 1) | ((r >> 1) & 1));
    f32x16 oacc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) oacc[db] = f32x16{};
#pragma unroll
    for (int blk = 0; blk < 2; ++blk)
#pragma unroll
        for (int kc = 0; kc < 2; ++kc)
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
                s16x4 half[2];
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int key = 32 * blk + 16 * kc + 8 * gl + 4 * h + tr_key;
                    half[h] = lds_read_tr16(vw + key * ROWP + 32 * db + tr_col);
                }
                const op_t va = __builtin_bit_cast(op_t, __builtin_shufflevector(half[0], half[1], 0, 1, 2, 3, 4, 5, 6, 7));
                oacc[db] = MfmaOp<T>::mma(va, pop[blk][kc], oacc[db]);
            }

    // combine the four wavefronts: (m, l, l_exact) and Oᵀ through LDS (the V
    // tiles are free once every wavefront has passed the barrier)
    __syncthreads();
    float* stash = reinterpret_cast<float*>(vt);
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int f = 0; f < 16; ++f) stash[((wave * NDB + db) * 16 + f) * 64 + lane] = oacc[db][f];
    s_ml[wave][0][lane] = mx;
    s_ml[wave][1][lane] = lsum;
    s_ml[wave][2][lane] = lex;
    __syncthreads();
    if (wave < NDB && live) {
        const int db = wave;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < 4; ++w) M = fmaxf(M, s_ml[w][0][lane]);
        float wt[4], lt = 0.0f, et = 0.0f;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            wt[w] = M == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(s_ml[w][0][lane] - M);
            lt += wt[w] * s_ml[w][1][lane];
            et += wt[w] * s_ml[w][2][lane];
        }
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
                for (int w = 0; w < 4; ++w) acc += wt[w] * stash[((w * NDB + db) * 16 + f) * 64 + lane];
                o8[e] = acc;
            }
            // head dims 32db + 16h + 8gl .. +7
            reinterpret_cast<u32x4*>(dst + 16 * h)[0] = *reinterpret_cast<const u32x4*>(&o8[0]);
            reinterpret_cast<u32x4*>(dst + 16 * h)[1] = *reinterpret_cast<const u32x4*>(&o8[4]);
        }
        if (db == 0 && gl == 0) {
            p.ws_m[pi] = M;
            p.ws_l[pi] = lt;
            p.ws_e[pi] = et;
        }
    }
}

// Merge of the chunks: one wavefront per output row; lanes read the chunk
// maxima and sums side by side, then accumulate the weighted partial outputs
// with the head dimension across lanes, eight chunks' loads in flight at once.
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
    dp.ws_e = dp.ws_l + int64_t(a.n_split) * rows;
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
    if constexpr (sizeof(T) == 2) {
        const int n_rg = (dp.R + kDecRowsMfma - 1) / kDecRowsMfma;
        attn_detail::log_launch("decode_mfma_kernel<%s, D=%d> grid=(%d, %lld, %d) block=%d Sk=%lld Sq=%lld",
                                attn_detail::dtype_name(a.dtype), D, a.n_split, (long long)(a.B * a.Hkv), n_rg,
                                kDecThreads, (long long)a.Sk, (long long)a.Sq);
        hipLaunchKernelGGL((decode_mfma_kernel<T, D>), dim3(unsigned(a.n_split), unsigned(a.B * a.Hkv), unsigned(n_rg)),
                           dim3(kDecThreads), 0, static_cast<hipStream_t>(a.stream), dp);
    } else {
        const int n_rg = (dp.R + kDecRows - 1) / kDecRows;
        attn_detail::log_launch("decode_split_kernel<%s, D=%d> grid=(%d, %lld, %d) block=%d Sk=%lld Sq=%lld",
                                attn_detail::dtype_name(a.dtype), D, a.n_split, (long long)(a.B * a.Hkv), n_rg,
                                kDecThreads, (long long)a.Sk, (long long)a.Sq);
        hipLaunchKernelGGL((decode_split_kernel<T, D>), dim3(unsigned(a.n_split), unsigned(a.B * a.Hkv), unsigned(n_rg)),
                           dim3(kDecThreads), 0, static_cast<hipStream_t>(a.stream), dp);
    }
    hipError_t e = hipGetLastError();
    if (e == hipSuccess) {
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
