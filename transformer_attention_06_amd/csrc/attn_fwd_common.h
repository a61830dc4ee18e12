// attn_fwd_common.h — device helpers of the fused attention forward kernel
// (attn_fwd_kernels.hip): MFMA wrappers, the transposing LDS read, the K/V
// tile swizzle, buffer resources and direct global->LDS loads, and the kernel
// parameter block.  Internal to the library.
#pragma once

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "attn_launch.h"

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));


template <typename T>
struct Elem;
template <>
struct Elem<__bf16> {
    static constexpr int KPL = 8;  // operand elements per lane per MFMA
    static constexpr int BN = 64;  // keys per K/V tile
    using op_t = bf16x8;
};
template <>
struct Elem<_Float16> {
    static constexpr int KPL = 8;
    static constexpr int BN = 64;
    using op_t = f16x8;
};
template <>
struct Elem<float> {
    static constexpr int KPL = 1;
    static constexpr int BN = 32;
    using op_t = float;
};

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma(f16x8 a, f16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma(float a, float b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// The same products as ordered inline assembly: the tile loop issues its
// MFMAs, operand reads and VALU work in a fixed interleaved order, and
// assembly statements are never reordered against each other or against
// memory operations.  "+v" accumulates in place; the zero-start form writes a
// fresh accumulator (early-clobber: no overlap with the operands).
__device__ __forceinline__ void mfma_acc(f32x16& c, const bf16x8& a, const bf16x8& b) {
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(c) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_acc(f32x16& c, const f16x8& a, const f16x8& b) {
    asm volatile("v_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+v"(c) : "v"(a), "v"(b));
}
// fp32 (a parity path, at the register limit at D = 128): the compiler's
// own MFMA, so that its hazard tracking covers any copy it inserts
__device__ __forceinline__ void mfma_acc(f32x16& c, const float& a, const float& b) {
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ void mfma_zero(f32x16& c, const bf16x8& a, const bf16x8& b) {
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(c) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_zero(f32x16& c, const f16x8& a, const f16x8& b) {
    asm volatile("v_mfma_f32_32x32x16_f16 %0, %1, %2, 0" : "=&v"(c) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_zero(f32x16& c, const float& a, const float& b) {
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, f32x16{}, 0, 0, 0);
}
// The output products with the accumulator in AGPRs (head dims above 160:
// one wavefront per SIMD, the accumulators beside a full set of VGPRs).
__device__ __forceinline__ void mfma_acc_a(f32x16& c, const bf16x8& a, const bf16x8& b) {
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_acc_a(f32x16& c, const f16x8& a, const f16x8& b) {
    asm volatile("v_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_acc_a(f32x16& c, const float& a, const float& b) { mfma_acc(c, a, b); }
// Sᵀ products with the Q operand (B) read from AGPRs, where those kernels
// keep it for the whole loop.
__device__ __forceinline__ void mfma_acc_qa(f32x16& c, const bf16x8& a, const bf16x8& b) {
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(c) : "v"(a), "a"(b));
}
__device__ __forceinline__ void mfma_acc_qa(f32x16& c, const f16x8& a, const f16x8& b) {
    asm volatile("v_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+v"(c) : "v"(a), "a"(b));
}
__device__ __forceinline__ void mfma_acc_qa(f32x16& c, const float& a, const float& b) { mfma_acc(c, a, b); }
__device__ __forceinline__ void mfma_zero_qa(f32x16& c, const bf16x8& a, const bf16x8& b) {
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(c) : "v"(a), "a"(b));
}
__device__ __forceinline__ void mfma_zero_qa(f32x16& c, const f16x8& a, const f16x8& b) {
    asm volatile("v_mfma_f32_32x32x16_f16 %0, %1, %2, 0" : "=&v"(c) : "v"(a), "a"(b));
}
__device__ __forceinline__ void mfma_zero_qa(f32x16& c, const float& a, const float& b) { mfma_zero(c, a, b); }
// a value made AGPR-resident here (the compiler keeps it there afterwards)
template <typename V>
__device__ __forceinline__ void to_agpr(V& x) {
    asm volatile("" : "+a"(x));
}
// Empty assembly statements that fix where VALU work happens in the stream:
// keep() marks values as needed at this point (computed no later); touch()
// marks a value as redefined here (work using it starts no earlier).
__device__ __forceinline__ void keep(float x) { asm volatile("" : : "v"(x)); }
__device__ __forceinline__ void keep_acc(const f32x16& x) { asm volatile("" : : "v"(x)); }
__device__ __forceinline__ void keep_acc_a(const f32x16& x) { asm volatile("" : : "a"(x)); }
__device__ __forceinline__ void touch(float& x) { asm volatile("" : "+v"(x)); }

template <typename OP, typename T>
__device__ __forceinline__ OP load_op(const T* p) {
    return *reinterpret_cast<const OP*>(p);
}

// Combine a value with the one held by lane l^32 (the other half of the
// same query row): one cross-half swap instead of an LDS permute.
__device__ __forceinline__ float max_xor32(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor32(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// The running max is only raised when a row's new tile max exceeds it by
// more than this many powers of two; otherwise the stale max is kept, the
// exponentials stay below 2^8 and the output accumulator needs no rescale.
constexpr float kRescaleLog2 = 8.0f;

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// Transposing LDS read: in each 16-lane group, lane 4j+q names an 8-byte
// piece (4 elements of one row); lane 4q+c receives element c of the pieces
// named by lanes 4j+q, j = 0..3 (a 4-row × 16-column block, transposed).
__device__ __forceinline__ s16x4 lds_read_tr16(const void* p) {
    typedef s16x4 __attribute__((address_space(3))) * lds_ptr;
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_ptr)(p));
}

// Sum of the two 16-bit probabilities in a packed pair, accumulated in fp32
// (dot product with (1, 1)): the row sum is taken over exactly the rounded
// values that enter the P·V product.
__device__ __forceinline__ float sum2(bf16x2 p, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(p, bf16x2{(__bf16)1.0f, (__bf16)1.0f}, acc, false);
}
__device__ __forceinline__ float sum2(f16x2 p, float acc) {
    return __builtin_amdgcn_fdot2(p, f16x2{(_Float16)1.0f, (_Float16)1.0f}, acc, false);
}

// A-operand row permutation: swap bits 2 and 3 of a 0..31 row index.
__device__ __forceinline__ int perm_row(int r) {
    return (r & 0x13) | ((r & 4) << 1) | ((r & 8) >> 1);
}

// Position (key within the tile, or head dim within a 32-wide block pair)
// held by accumulator register f (0..16*blocks-1) of a lane in half g.
__host__ __device__ constexpr int kidx(int f, int g) {
    return 32 * (f >> 4) + 16 * ((f >> 3) & 1) + 8 * g + (f & 7);
}

struct KParams {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    float* lse;
    const int32_t* pad_lens;
    int S, Hq, Hkv, group, n_qb, n_units, xcd_chunk;
    int64_t q_bstride, kv_bstride;  // elements per batch
    const int32_t* cu;              // packed sequences: offsets cu[0..B] into T rows, or null
    int total;                      // T (packed sequences; S is then the longest length)
    float sl2;                      // scale * log2(e)
    const int32_t* rope_pos;        // (B, S) positions, or null for 0..S-1
    double rope_r1;                 // rho = base^(-2/D): theta_{i+1} / theta_i
    // explicit mask tensor (Bm, Hm, S, S): additive in the input type or one
    // byte per entry; mask_b / mask_h are 1 when it has a batch / head
    // dimension of B / Hq
    const void* mask;
    int mask_b, mask_h;
    float inv_scale;                // 1 / scale: the additive mask in raw score units
};

// Rotary embedding: cos and sin of position × theta_i, from f = theta_i / 2π.
// The angle in turns is reduced to [-1/2, 1/2] in fp64, which is exact
// enough for any int32 position; the 16-bit types then use the hardware sine
// and cosine of a turn count (their error is far below the rounding of the
// rotated value to 16 bits), fp32 the full-precision library sincos.
template <typename T>
__device__ __forceinline__ void rope_cs(int pos, double f, float& c, float& s) {
    const double turns = double(pos) * f;
    const double r = turns - __builtin_rint(turns);
    if constexpr (sizeof(T) == 2) {
        const float rf = float(r);
        s = __builtin_amdgcn_sinf(rf);
        c = __builtin_amdgcn_cosf(rf);
    } else {
        sincosf(float(r * 6.283185307179586476925), &s, &c);
    }
}

template <typename T>
__device__ __forceinline__ T to_t(float x) {
    return static_cast<T>(x);
}

// XOR swizzle of the 16-byte slots of a K/V tile row (NS slots per row).
// With 64 LDS banks, this makes the three access patterns of the kernel
// conflict-free: 16-lane row writes, the K-operand reads (16 permuted rows,
// one slot each) and the transposing V reads (4 consecutive rows, 32 bytes
// each, two 16-lane groups side by side).
template <int NS>
__device__ __forceinline__ int swz(int row) {
    if constexpr (NS >= 16)
        return ((row & 3) << 2) | ((row >> 2) & 3);
    else
        return (((row >> 1) & 1) << 2) | ((row >> 2) & 3);
}

typedef int i32x4 __attribute__((ext_vector_type(4)));

// Buffer resource words for [base, base + bytes) (gfx9 default data format);
// loads at offsets at or past the end return zero.
__device__ __forceinline__ i32x4 rsrc_words(const void* base, uint32_t bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    return i32x4{int(uint32_t(a)), int(uint32_t(a >> 32) & 0xffff), int(bytes), 0x00020000};
}

// One 16-byte global load per lane, written to LDS at lds_byte + 16·lane
// (buffer_load_dwordx4 with LDS destination; M0 holds the LDS address).
// Issued as inline assembly on purpose: the compiler then does not track
// these LDS writes and inserts no waits for them before unrelated LDS reads
// (it cannot prove the tile being read differs from the tile being loaded).
// Every read of a loaded tile is ordered explicitly instead: the loading
// wave waits vmcnt(0), then a workgroup barrier.  No other code in the kernel
// uses M0.
__device__ __forceinline__ void lds_dma16(const i32x4& rs, uint32_t lds_byte, uint32_t voff) {
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :
                 : "s"(lds_byte), "v"(voff), "s"(rs)
                 : "memory");
}

// s_waitcnt vmcnt(n) for 0 <= n < 16 (n a constant after unrolling), also
// a compiler barrier for memory operations: the direct global->LDS loads
// are assembly the compiler does not track.
__device__ __forceinline__ void wait_vmcnt(int n) {
    switch (n) {
        case 0: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
        case 1: asm volatile("s_waitcnt vmcnt(1)" ::: "memory"); break;
        case 2: asm volatile("s_waitcnt vmcnt(2)" ::: "memory"); break;
        case 3: asm volatile("s_waitcnt vmcnt(3)" ::: "memory"); break;
        case 4: asm volatile("s_waitcnt vmcnt(4)" ::: "memory"); break;
        case 5: asm volatile("s_waitcnt vmcnt(5)" ::: "memory"); break;
        case 6: asm volatile("s_waitcnt vmcnt(6)" ::: "memory"); break;
        case 7: asm volatile("s_waitcnt vmcnt(7)" ::: "memory"); break;
        case 8: asm volatile("s_waitcnt vmcnt(8)" ::: "memory"); break;
        case 9: asm volatile("s_waitcnt vmcnt(9)" ::: "memory"); break;
        case 10: asm volatile("s_waitcnt vmcnt(10)" ::: "memory"); break;
        case 11: asm volatile("s_waitcnt vmcnt(11)" ::: "memory"); break;
        case 12: asm volatile("s_waitcnt vmcnt(12)" ::: "memory"); break;
        case 13: asm volatile("s_waitcnt vmcnt(13)" ::: "memory"); break;
        case 14: asm volatile("s_waitcnt vmcnt(14)" ::: "memory"); break;
        default: asm volatile("s_waitcnt vmcnt(15)" ::: "memory"); break;
    }
}

}  // namespace
