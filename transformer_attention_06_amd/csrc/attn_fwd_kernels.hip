// attn_fwd_kernels.hip — fused attention forward for gfx950 (MI355X).
//
// One workgroup (4 wavefronts of 64 lanes) owns one (batch, query head,
// 128-row query block); each wavefront owns 32 query rows.  K/V tiles of BN
// keys stream through double-buffered LDS; the score tile, the online-softmax
// state and the output accumulator never leave registers, so the S×S score
// matrix never reaches device memory ("ops-transformer：Transformer算子融合与
// 推理加速实战" §2.2 structural fusion, §3.2 blockwise loop nest with a running
// local max and sum, §2.3 prefetching the next block while the current one is
// computed).
//
// Both products run on MFMA, computed TRANSPOSED so that every lane owns one
// query row:
//     Sᵀ (keys × rows)  = K · Qᵀ      A = K tile (LDS),  B = Q (registers)
//     Oᵀ (dims × rows) += Vᵀ · Pᵀ     A = Vᵀ tile (LDS), B = P (registers)
// With the 32×32 MFMA accumulator layout, lane l holds column l%32 (= one
// query row) and 16 rows of the tile, so the softmax row max and row sum are
// in-lane reductions plus one exchange with lane l^32, the P operand of the
// second product is formed from the first product's accumulators without any
// data movement, and the rescale of the output accumulator by the running-max
// correction is a per-lane scalar.  The A operands are loaded with a fixed
// row permutation (bits 2 and 3 of the row index swapped) so that each lane's
// registers cover 8 consecutive keys / head dims: P packs straight into MFMA
// operands and the output is stored as 16-byte vectors.  K and V both sit in
// LDS row-major (key-major, as in memory); the Vᵀ operand is read with the
// gfx950 transposing LDS read (ds_read_b64_tr_b16), whose 4×16 transpose per
// 16-lane group lines up with the same bit-2/3 row permutation.
//
// Precision ("ops-transformer…" §2.4): bf16/fp16 storage and MFMA inputs, fp32
// accumulation, fp32 running max / sum, output rounded to the storage type at
// the end.  Scores are scaled by scale·log2(e) so the exponentials are exp2.
// The fp32 path uses the fp32 MFMA and keeps P in fp32.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "attn_fwd.h"
#include "attn_launch.h"

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int BM = attn_detail::kBlockM;  // 128 query rows per workgroup
static_assert(BM == 4 * 32, "4 wavefronts x 32 rows");

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

template <typename OP, typename T>
__device__ __forceinline__ OP load_op(const T* p) {
    return *reinterpret_cast<const OP*>(p);
}

// Buffer resource over [base, base + bytes): loads at offsets at or past the
// end return zero, which zero-fills K/V rows beyond the sequence end without
// branches.  Word 3 is the gfx9-family default data format.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, int(bytes), 0x00020000);
}
__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, int(voff), int(soff), 0);
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
    float sl2;                      // scale * log2(e)
};

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

template <typename T>
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t r, T* lds_dst, uint32_t voff) {
    // one 16-byte global load per lane, written to lds_dst + 16 * lane
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)(lds_dst), 16,
                                             voff, 0, 0, 0);
}

// 16-bit instances keep two wavefronts per SIMD (two workgroups per CU); the
// fp32 instances hold twice the operand registers and run one.
template <typename T, int D, bool CAUSAL, bool PAD, bool LSE>
__global__ __launch_bounds__(kThreads, sizeof(T) == 2 ? 2 : 1) void attn_fwd_kernel(KParams p) {
    using E = Elem<T>;
    using op_t = typename E::op_t;
    constexpr int KPL = E::KPL;
    constexpr int BN = E::BN;
    constexpr int ES = int(sizeof(T));
    constexpr int CH = 16 / ES;            // elements per 16-byte slot
    constexpr int NS = D / CH;             // slots per tile row
    constexpr int ROW_B = D * ES;          // bytes per tile row
    constexpr int TILE_E = BN * D;         // elements per K (or V) tile
    constexpr int NLD = BN * ROW_B / 4096; // 1 KiB direct loads per wave per tile
    static_assert(NLD * 4096 == BN * ROW_B, "tile split into 1 KiB wave loads");
    constexpr int NC = D / (2 * KPL);      // MFMA steps along D (Sᵀ)
    constexpr int NBLK = BN / 32;          // 32-key blocks per tile
    constexpr int NKC = BN / (2 * KPL);    // MFMA steps along keys (Oᵀ)
    constexpr int NDB = D / 32;            // 32-dim blocks of O

    // K and V tiles, each double-buffered, each row-major [BN][D] with
    // swizzled slots.  Four distinct objects: the compiler can then see that
    // a tile being read never aliases the tiles whose loads are in flight,
    // and does not wait for those loads before the reads.
    __shared__ __attribute__((aligned(1024))) T kbuf0[TILE_E];
    __shared__ __attribute__((aligned(1024))) T kbuf1[TILE_E];
    __shared__ __attribute__((aligned(1024))) T vbuf0[TILE_E];
    __shared__ __attribute__((aligned(1024))) T vbuf1[TILE_E];

    // ---- work decomposition ------------------------------------------------
    // Workgroup i runs on XCD i % 8.  Logical units (batch, kv head, query
    // head) are split into 8 contiguous ranges, one per XCD, so the query
    // heads sharing a K/V head share that XCD's L2.  Under causal masking the
    // query blocks are ordered heaviest first for the first half of the
    // launch and lightest first for the second half, so the two workgroups
    // that the dispatcher co-schedules on a CU (i and i + grid/2) carry equal
    // total work when the whole grid is resident at once.
    const int wg = blockIdx.x;
    int unit, qb_rank;
    if (p.xcd_chunk > 0) {
        const int xcd = wg & 7, local = wg >> 3;
        qb_rank = local / p.xcd_chunk;
        unit = xcd * p.xcd_chunk + local % p.xcd_chunk;
    } else {
        qb_rank = wg / p.n_units;
        unit = wg % p.n_units;
    }
    int qb = qb_rank;
    if (CAUSAL) {
        const int half = (p.n_qb + 1) >> 1;
        qb = qb_rank < half ? p.n_qb - 1 - qb_rank : qb_rank - half;
    }
    const int jg = unit % p.group;
    const int bg = unit / p.group;
    const int g = bg % p.Hkv;
    const int b = bg / p.Hkv;
    const int hq = g * p.group + jg;

    const int S = p.S;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int r = lane & 31;
    const int gl = lane >> 5;
    const int q0 = qb * BM;
    const int wrow0 = q0 + wave * 32;
    const int qrow = wrow0 + r;

    const int64_t qstride = int64_t(p.Hq) * D;
    const int64_t kvstride = int64_t(p.Hkv) * D;
    const T* qbase = static_cast<const T*>(p.q) + int64_t(b) * p.q_bstride + int64_t(hq) * D;
    const T* kbase = static_cast<const T*>(p.k) + int64_t(b) * p.kv_bstride + int64_t(g) * D;
    const T* vbase = static_cast<const T*>(p.v) + int64_t(b) * p.kv_bstride + int64_t(g) * D;

    // ---- Q tile: MFMA B operands, resident for the whole loop ------------
    op_t qv[NC];
    if (qrow < S) {
        const T* qr = qbase + int64_t(qrow) * qstride;
#pragma unroll
        for (int c = 0; c < NC; ++c) qv[c] = load_op<op_t>(qr + c * 2 * KPL + gl * KPL);
    } else {
#pragma unroll
        for (int c = 0; c < NC; ++c) qv[c] = op_t{};
    }

    // ---- key range ----------------------------------------------------------
    int key_lim = S;
    if (PAD) {
        const int L = p.pad_lens[b];
        key_lim = L < 0 ? 0 : (L > S ? S : L);
    }
    int key_end = key_lim;
    if (CAUSAL) key_end = key_end < q0 + BM ? key_end : q0 + BM;
    const int n_tiles = (key_end + BN - 1) / BN;

    // ---- tile loads: global -> LDS directly -------------------------------
    // Buffer resources cover this (batch, kv head) slice; rows at or past S
    // read as zero.  Wave w fills bytes [w·NLD KiB, (w+1)·NLD KiB) of each
    // tile; lane l writes the 16-byte slot at l·16 of its KiB, i.e. row
    // (KiB offset + 16 l) / ROW_B at physical slot p, which holds logical
    // slot p ^ swz(row) of that key row.
    const uint32_t kv_bytes = uint32_t((int64_t(S) * kvstride - int64_t(g) * D) * int64_t(ES));
    const __amdgpu_buffer_rsrc_t krs = make_rsrc(kbase, kv_bytes);
    const __amdgpu_buffer_rsrc_t vrs = make_rsrc(vbase, kv_bytes);
    const uint32_t row_bytes = uint32_t(kvstride * int64_t(ES));
    uint32_t ld_off[NLD];
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
        const int byte = (wave * NLD + i) * 1024 + lane * 16;
        const int row = byte / ROW_B;
        const int lslot = ((byte % ROW_B) / 16) ^ swz<NS>(row);
        ld_off[i] = uint32_t(row) * row_bytes + uint32_t(lslot * 16);
    }
    auto issue = [&](__amdgpu_buffer_rsrc_t rs, T* dst, int kb) {
        const uint32_t tile_off = uint32_t(kb) * row_bytes;
#pragma unroll
        for (int i = 0; i < NLD; ++i) lds_dma16(rs, dst + ((wave * NLD + i) * 1024) / ES, ld_off[i] + tile_off);
    };

    // ---- per-lane LDS read offsets (elements, within a tile) ---------------
    const int prow = perm_row(r);
    const int xk = swz<NS>(prow);  // swizzle of every K row this lane reads (row ≡ prow mod 16)
    // transposing V reads: lane addresses key (r & 15) >> 2 of a 4-key group,
    // head dims 16·(r >> 4) + 4·swap01(r & 3) .. +3 of each 32-dim block
    const int tr_key = (r & 15) >> 2;
    const int tr_col = 16 * (r >> 4) + 4 * (((r & 1) << 1) | ((r >> 1) & 1));
    // element offset of this lane's transposing read for (db, h) at kc = 0;
    // key 16·kc + k has the swizzle of k (16·kc ≡ 0 mod 16), so kc only adds
    // the constant 16·kc·D
    int v_off[NDB][2];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int key = 8 * gl + 4 * h + tr_key;
            const int col = 32 * db + tr_col;
            v_off[db][h] = key * D + (((col / CH) ^ swz<NS>(key)) * CH) + col % CH;
        }

    // ---- online-softmax state ----------------------------------------------
    f32x16 oacc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) oacc[db] = f32x16{};
    float m_run = -INFINITY;  // running max of scale*log2(e)*score
    float l_run = 0.0f;       // running sum of the rounded P (this lane's half of the keys)
    float l_lse = 0.0f;       // running sum of the unrounded P, for the LSE output
    const float sl2 = p.sl2;

    // Sᵀ = K · Qᵀ for this wave's 32 rows, K from an LDS tile
    auto gemm1 = [&](const T* ks, f32x16 (&sacc)[NBLK]) {
#pragma unroll
        for (int blk = 0; blk < NBLK; ++blk) sacc[blk] = f32x16{};
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const int col = c * 2 * KPL + gl * KPL;
            const int off = (((col / CH) ^ xk) * CH) + col % CH;
#pragma unroll
            for (int blk = 0; blk < NBLK; ++blk) {
                const op_t a = load_op<op_t>(ks + (prow + 32 * blk) * D + off);
                sacc[blk] = mfma(a, qv[c], sacc[blk]);
            }
        }
    };

    // Mask, running max and (rare) rescale for the scores of the tile at kb.
    auto softmax_max = [&](f32x16 (&sacc)[NBLK], int kb) {
        // mask: keys past the valid length, and keys after the row (causal)
        const bool need_mask = (kb + BN > key_lim) || (CAUSAL && kb + BN - 1 > wrow0);
        if (need_mask) {
#pragma unroll
            for (int blk = 0; blk < NBLK; ++blk)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int key = kb + kidx(16 * blk + i, gl);
                    const bool ok = key < key_lim && (!CAUSAL || key <= qrow);
                    if (!ok) sacc[blk][i] = -INFINITY;
                }
        }
        // row max over this lane's 16·NBLK scores in four independent chains
        float mp[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
        for (int blk = 0; blk < NBLK; ++blk)
#pragma unroll
            for (int i = 0; i < 16; ++i) mp[i & 3] = fmaxf(mp[i & 3], sacc[blk][i]);
        float mx = fmaxf(fmaxf(mp[0], mp[1]), fmaxf(mp[2], mp[3]));
        mx = max_xor32(mx) * sl2;
        // raise the running max only when some row of the wave needs it
        if (__builtin_amdgcn_ballot_w64(mx > m_run + kRescaleLog2) != 0) {
            const float m_new = fmaxf(m_run, mx);
            const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
            l_run *= alpha;
            if constexpr (LSE) l_lse *= alpha;
#pragma unroll
            for (int db = 0; db < NDB; ++db) oacc[db] *= alpha;
            m_run = m_new;
        }
    };

    // Exponentials, P packed into MFMA operands, row sums.
    auto softmax_exp = [&](const f32x16 (&sacc)[NBLK], op_t (&pb)[NKC]) {
        const float m_use = (m_run == -INFINITY) ? 0.0f : m_run;
        // row sums in four independent chains
        float rs[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        float rl[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int f = 0; f < 16 * NBLK; ++f) {
            const float pv = __builtin_amdgcn_exp2f(fmaf(sacc[f >> 4][f & 15], sl2, -m_use));
            if constexpr (KPL == 1) {
                pb[f] = pv;
                rs[f & 3] += pv;
            } else {
                pb[f / KPL][f % KPL] = to_t<T>(pv);
                if constexpr (LSE) rl[f & 3] += pv;
            }
        }
        if constexpr (KPL == 1) {
#pragma unroll
            for (int i = 0; i < 4; ++i) rl[i] = rs[i];
        } else {
            typedef T t2 __attribute__((ext_vector_type(2)));
#pragma unroll
            for (int kc = 0; kc < NKC; ++kc)
#pragma unroll
                for (int e = 0; e < KPL; e += 2)
                    rs[(kc * KPL + e) / 2 & 3] = sum2(t2{pb[kc][e], pb[kc][e + 1]}, rs[(kc * KPL + e) / 2 & 3]);
        }
        l_run += (rs[0] + rs[1]) + (rs[2] + rs[3]);
        if constexpr (LSE) l_lse += (rl[0] + rl[1]) + (rl[2] + rl[3]);
    };

    // Oᵀ += Vᵀ · Pᵀ, V from an LDS tile
    auto gemm2 = [&](const T* vs, const op_t (&pb)[NKC]) {
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc) {
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
                op_t a;
                if constexpr (KPL == 1) {
                    const int key = kidx(kc, gl);
                    const int col = 32 * db + prow;
                    a = vs[key * D + (((col / CH) ^ swz<NS>(key)) * CH) + col % CH];
                } else {
                    s16x4 half[2];
#pragma unroll
                    for (int h = 0; h < 2; ++h) half[h] = lds_read_tr16(vs + 16 * kc * D + v_off[db][h]);
                    a = __builtin_bit_cast(op_t, __builtin_shufflevector(half[0], half[1], 0, 1, 2, 3, 4, 5, 6, 7));
                }
                oacc[db] = mfma(a, pb[kc], oacc[db]);
            }
        }
    };

    // One tile: Sᵀ from K, softmax, O += P·V from V.  (A variant that
    // overlapped the next tile's Sᵀ with this tile's softmax needed a second
    // score tile in registers and ran slower at two wavefronts per SIMD.)
    auto step = [&](int kb, const T* ks, const T* vs) {
        if (CAUSAL && kb > wrow0 + 31) return;  // no key of the tile is visible to this wave
        f32x16 sacc[NBLK];
        gemm1(ks, sacc);
        softmax_max(sacc, kb);
        op_t pb[NKC];
        softmax_exp(sacc, pb);
        gemm2(vs, pb);
    };

    // ---- main loop ----------------------------------------------------------
    // Tile j computes from buffer j % 2 while tile j+1 loads into the other;
    // one barrier per tile publishes the loads and releases the buffer.
    if (n_tiles > 0) {
        issue(krs, kbuf0, 0);
        issue(vrs, vbuf0, 0);
    }
    // All loads issued so far (Q and the first tile) are complete here on
    // every path; saying so keeps the loop free of waits on them.
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    __syncthreads();
    for (int j = 0; j < n_tiles; j += 2) {
        const int kb = j * BN;
        if (j + 1 < n_tiles) {
            issue(krs, kbuf1, kb + BN);
            issue(vrs, vbuf1, kb + BN);
        }
        step(kb, kbuf0, vbuf0);
        __builtin_amdgcn_s_waitcnt(0x0F70);  // this wave's loads landed
        __syncthreads();
        if (j + 1 >= n_tiles) break;
        if (j + 2 < n_tiles) {
            issue(krs, kbuf0, kb + 2 * BN);
            issue(vrs, vbuf0, kb + 2 * BN);
        }
        step(kb + BN, kbuf1, vbuf1);
        __builtin_amdgcn_s_waitcnt(0x0F70);
        __syncthreads();
    }

    // ---- epilogue: normalise, store O (and LSE) ---------------------------
    const float l_tot = sum_xor32(l_run);
    const float l_e = LSE ? sum_xor32(l_lse) : 0.0f;
    const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
    if (qrow < S) {
        T* orow = static_cast<T*>(p.o) + int64_t(b) * p.q_bstride + int64_t(qrow) * qstride +
                  int64_t(hq) * D;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                T vals[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) vals[e] = to_t<T>(oacc[db][8 * h + e] * inv);
                T* dst = orow + 32 * db + 16 * h + 8 * gl;
                if constexpr (sizeof(T) == 2) {
                    *reinterpret_cast<u32x4*>(dst) = *reinterpret_cast<const u32x4*>(vals);
                } else {
                    reinterpret_cast<u32x4*>(dst)[0] = reinterpret_cast<const u32x4*>(vals)[0];
                    reinterpret_cast<u32x4*>(dst)[1] = reinterpret_cast<const u32x4*>(vals)[1];
                }
            }
        if (LSE && gl == 0) {
            const float lse = l_e > 0.0f ? (m_run + __builtin_amdgcn_logf(l_e)) * 0.69314718055994530942f
                                         : -INFINITY;
            p.lse[(int64_t(b) * p.Hq + hq) * S + qrow] = lse;
        }
    }
}

template <typename T, int D, bool CAUSAL, bool PAD, bool LSE>
int launch_t(const attn_detail::LaunchArgs& a) {
    KParams kp;
    kp.q = a.q;
    kp.k = a.k;
    kp.v = a.v;
    kp.o = a.o;
    kp.lse = a.lse;
    kp.pad_lens = a.pad_lens;
    kp.S = int(a.S);
    kp.Hq = int(a.Hq);
    kp.Hkv = int(a.Hkv);
    kp.group = int(a.Hq / a.Hkv);
    kp.n_qb = int((a.S + BM - 1) / BM);
    kp.n_units = int(a.B * a.Hq);
    kp.xcd_chunk = (kp.n_units % 8 == 0) ? kp.n_units / 8 : 0;
    kp.q_bstride = a.S * a.Hq * a.D;
    kp.kv_bstride = a.S * a.Hkv * a.D;
    kp.sl2 = a.scale * 1.44269504088896340736f;
    const int64_t n_wg = int64_t(kp.n_qb) * kp.n_units;
    hipLaunchKernelGGL((attn_fwd_kernel<T, D, CAUSAL, PAD, LSE>), dim3(unsigned(n_wg)), dim3(kThreads), 0,
                       static_cast<hipStream_t>(a.stream), kp);
    const hipError_t e = hipGetLastError();
    if (e == hipSuccess) return ATTN_OK;
    if (e == hipErrorNoBinaryForGpu || e == hipErrorInvalidDeviceFunction) return ATTN_ERR_DEVICE;
    return ATTN_ERR_LAUNCH;
}

template <typename T, int D, bool LSE>
int launch_l(const attn_detail::LaunchArgs& a) {
    if (a.causal) return a.padded ? launch_t<T, D, true, true, LSE>(a) : launch_t<T, D, true, false, LSE>(a);
    return a.padded ? launch_t<T, D, false, true, LSE>(a) : launch_t<T, D, false, false, LSE>(a);
}

template <typename T, int D>
int launch_d(const attn_detail::LaunchArgs& a) {
    return a.lse != nullptr ? launch_l<T, D, true>(a) : launch_l<T, D, false>(a);
}

template <typename T>
int launch_dtype(const attn_detail::LaunchArgs& a) {
    return a.D == 64 ? launch_d<T, 64>(a) : launch_d<T, 128>(a);
}

}  // namespace

namespace attn_detail {

int launch(const LaunchArgs& a) {
    switch (a.dtype) {
        case ATTN_BF16: return launch_dtype<__bf16>(a);
        case ATTN_F16: return launch_dtype<_Float16>(a);
        default: return launch_dtype<float>(a);
    }
}

}  // namespace attn_detail
