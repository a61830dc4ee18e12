// attn_masked_kernels.hip — fused attention forward with an explicit mask
// tensor, and the general-head-dim attention (gfx950).
//
// "CANN-ATB图优化-昇腾NPU怎么把PyTorch计算图改造成融合算子" Pattern 2 fuses
// Q·Kᵀ → Scale → Mask → Softmax → ·V into FlashAttention(Q, K, V, mask,
// scale), and the ATB engineering guide (hwcomputing.csdn.net/
// 6a59a88310ee7a33f28e5ce9) §8.2 hands the mask to the operator as one more
// FP16 input tensor.  Here the mask M (1 or B, 1 or Hq, S, S) is added to the
// scaled scores, in the input type (-inf hides a key), or given as one byte
// per entry (nonzero: the key takes part).  The same kernel without a mask
// serves head dims other than 64 and 128 ("CANN-ops-transformer和ATB…" gates
// head_dim on multiples of 16), the head dim padded to a multiple of 32 in
// registers and LDS only.
//
// A group of 4 wavefronts owns one (batch, query head, 128-row query block);
// each wavefront owns 32 query rows, one per lane, in the transposed MFMA
// form of the prefill kernel: Sᵀ = K·Qᵀ and Oᵀ += Vᵀ·Pᵀ on 32x32x16 MFMA.
// Up to head dim 160 a workgroup holds two such groups splitting the block's
// key tiles (merged through LDS at the end), and under causal masking a
// workgroup runs the heaviest and the lightest block in turn.  Per 64-key
// tile every lane loads the 32 mask values of its row that its score
// registers hold (four runs of 8 consecutive keys, thanks to the permuted K
// order); the K and V tiles are staged per group in LDS (V read back with the
// transposing LDS read), double-buffered where LDS allows, and the next
// tile's K, V and mask loads are in flight while the current tile is
// computed ("ops-transformer：Transformer算子融合与推理加速实战" §2.3: prefetch
// the next block during the current one).  The online softmax keeps fp32
// running max and sums per row (§3.2) and rescales the output accumulator
// whenever the max rises.  Unlike the tuned D = 64/128 kernel the MFMAs and
// the softmax are not interleaved by hand.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "attn_fwd.h"
#include "attn_launch.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

template <typename T>
struct Op;
template <>
struct Op<__bf16> {
    using op_t = bf16x8;
    static __device__ __forceinline__ f32x16 mma(op_t a, op_t b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
};
template <>
struct Op<_Float16> {
    using op_t = f16x8;
    static __device__ __forceinline__ f32x16 mma(op_t a, op_t b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    }
};

constexpr int kMThreads = 256;  // 4 wavefronts
constexpr int kMRows = 128;     // query rows per workgroup
constexpr int kMKeys = 64;      // keys per tile

struct MParams {
    const void* q;
    const void* k;
    const void* v;
    const void* mask;  // (Bm, Hm, S, S) in the input type
    void* o;
    float* lse;
    int S, Hq, Hkv, group, n_qb, D;
    const int32_t* pad_lens;  // key padding (int32[B]) or null
    int pair;  // causal: heavy/light query blocks paired in one workgroup
    int mask_b, mask_h;  // 1 when the mask has a batch (head) dimension of B (Hq)
    float sl2;           // scale * log2(e)
};

// A-operand row permutation (swap bits 2 and 3 of a 0..31 row index) and the
// key / head dim that accumulator register f of a lane in half g then holds
// within its 32-block: 16·((f >> 3) & 1) + 8·g + (f & 7).
__device__ __forceinline__ int perm_row(int r) { return (r & 0x13) | ((r & 4) << 1) | ((r & 8) >> 1); }
__device__ __forceinline__ int acc_pos(int f, int g) { return 16 * ((f >> 3) & 1) + 8 * g + (f & 7); }

// Transposing LDS read: in each 16-lane group, lane 4j+q names an 8-byte
// piece (4 elements of one row); lane 4q+c receives element c of the pieces
// named by lanes 4j+q, j = 0..3.
__device__ __forceinline__ s16x4 lds_read_tr16(const void* ptr) {
    typedef s16x4 __attribute__((address_space(3))) * lds_ptr;
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_ptr)(ptr));
}

// value held by lane l ^ 32
__device__ __forceinline__ float xor32(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float((threadIdx.x & 32) ? r[0] : r[1]);
}

// DP: the head dimension padded to a multiple of 32 (the tile width); the
// real head dimension p.D (a multiple of 16, at most DP) sets the strides,
// and head-dim chunks at or past it are read as zeros and not written.
// MK: 0 no mask tensor; 1 an additive mask tensor whose rows are 16-byte
// aligned (S a multiple of 8: 16-byte loads); 2 the same with unaligned rows
// (element loads); 3 a boolean mask (one byte per entry, nonzero: the key
// takes part) with 8-byte aligned rows (8-byte loads); 4 the same unaligned
// (byte loads).  EXACT: D == DP, known at compile time (no head-dim
// guards).
//
// Head dims up to 160 run two groups of four wavefronts per workgroup (NG =
// 2): both groups take the same query block, group 0 its first half of the
// key tiles and group 1 the second half, each with its own LDS tiles, and
// the two partial softmax states (m, l, O) are merged through LDS at the end
// of the block ("ops-transformer…" §3.2's recurrence applied to two key
// ranges).  Wider head dims run one group (their registers need one
// wavefront per SIMD).
template <int DP>
struct MGroups {
    static constexpr int value = DP <= 160 ? 2 : 1;
};

template <typename T, int DP, bool CAUSAL, int MK, bool EXACT>
__global__ __launch_bounds__(kMThreads * MGroups<DP>::value, 1) void masked_kernel(MParams p) {
    using op_t = typename Op<T>::op_t;
    constexpr bool MASK = MK != 0;
    constexpr bool BMASK = MK >= 3;  // boolean mask
    constexpr int NG = MGroups<DP>::value;
    constexpr int NC = DP / 16;                    // MFMA steps along the head dim for Sᵀ
    constexpr int NDB = DP / 32;                   // 32-dim blocks of Oᵀ
    constexpr int ROWP = DP + 8;                   // LDS row pitch of the K and V tiles (elements)
    constexpr int CPR = DP / 8;                    // 16-byte chunks per (padded) row
    constexpr int NVL = kMKeys * CPR / kMThreads;  // V chunks per thread
    static_assert(NVL * kMThreads == kMKeys * CPR, "V tile split over a group");
    constexpr int TILE = kMKeys * ROWP;            // elements per K (or V) tile
    // per group: V tile, then K tile; after a block the region holds group
    // 1's partial output for the merge
    // two K/V buffers per group where LDS holds them (one barrier per tile),
    // else one (two barriers per tile)
    constexpr int NBUF = (NG * 2 * 2 * TILE * int(sizeof(T)) + 3072 <= 160 * 1024) ? 2 : 1;
    __shared__ __attribute__((aligned(16))) T lds[NG * NBUF * 2 * TILE];
    __shared__ float s_ml[4][3][64];
    static_assert(NG == 1 || 4 * (DP / 32) * 16 * 64 * 4 <= int(sizeof(lds)), "merge stash fits the tiles");

    // Under causal masking, when pairing is on (p.pair: always with two
    // groups, else when the launch keeps two workgroups on every CU anyway),
    // a workgroup runs two query blocks one after the other, the heaviest and the lightest remaining
    // (n_qb-1-i, then i), so every workgroup streams the same number of key
    // tiles and the last query block does not set the kernel's time alone.
    // Otherwise one block per workgroup, heaviest first.
    int nseg = 1, qb0 = CAUSAL ? p.n_qb - 1 - int(blockIdx.x) : int(blockIdx.x), qb1 = -1;
    if (CAUSAL && p.pair) {
        qb0 = p.n_qb - 1 - int(blockIdx.x);
        qb1 = int(blockIdx.x) < qb0 ? int(blockIdx.x) : -1;
        nseg = qb1 >= 0 ? 2 : 1;
    }
    const int hq = blockIdx.y, b = blockIdx.z;
    const int g = hq / p.group;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int w4 = wave & 3;                  // 32-row slice of the query block
    const int grp = NG == 2 ? wave >> 2 : 0;  // key half of the block
    const int gtid = tid & (kMThreads - 1);   // thread index within the group
    T* const gbuf = lds + grp * NBUF * 2 * TILE;  // this group's buffers: V tile, then K tile, per buffer
    const int r = lane & 31, gl = lane >> 5;
    const int S = p.S;
    const int D = EXACT ? DP : p.D;
    int key_lim = S;  // keys at or past this are hidden (key padding)
    if (p.pad_lens) {
        const int L = p.pad_lens[b];
        key_lim = L < 0 ? 0 : (L > S ? S : L);
    }
    for (int sg = 0; sg < nseg; ++sg) {
        const int qb = sg == 0 ? qb0 : qb1;
        const int q0 = qb * kMRows;
        const int qrow = q0 + w4 * 32 + r;
        const bool live = qrow < S;

        const int64_t qstride = int64_t(p.Hq) * D;
        const int64_t kvstride = int64_t(p.Hkv) * D;
        const T* kb = static_cast<const T*>(p.k) + int64_t(b) * S * kvstride + int64_t(g) * D;
        const T* vb = static_cast<const T*>(p.v) + int64_t(b) * S * kvstride + int64_t(g) * D;
        const int64_t plane = int64_t(p.mask_b ? b : 0) * (p.mask_h ? p.Hq : 1) + (p.mask_h ? hq : 0);
        const int64_t mrow_off = (plane * S + (live ? qrow : 0)) * int64_t(S);
        const T* mrow = MASK && !BMASK ? static_cast<const T*>(p.mask) + mrow_off : nullptr;
        const uint8_t* mrow8 = BMASK ? static_cast<const uint8_t*>(p.mask) + mrow_off : nullptr;

        // Q operand: the lane's row, head dims 16c + 8gl .. +7
        op_t qop[NC];
        const T* qr = static_cast<const T*>(p.q) + (int64_t(b) * S + (live ? qrow : S - 1)) * qstride +
                      int64_t(hq) * D + 8 * gl;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            // unconditional load from a valid address (row S-1 for rows past
            // S, whose results are never written; chunk 0 for head-dim chunks
            // past D, zeroed by the select): no branch, all loads in flight
            const bool in_d = EXACT || 16 * c + 8 * gl < D;
            const op_t x = *reinterpret_cast<const op_t*>(qr + (in_d ? 16 * c : 0));
            qop[c] = in_d ? x : op_t{};
        }

        const int kend = CAUSAL ? (key_lim < q0 + kMRows ? key_lim : q0 + kMRows) : key_lim;
        const int ntile = (kend + kMKeys - 1) / kMKeys;
        const int tr_key = (r & 15) >> 2;
        const int tr_col = 16 * (r >> 4) + 4 * (((r & 1) << 1) | ((r >> 1) & 1));
        float m_run = -INFINITY, l_run = 0.0f, l_ex = 0.0f;
        f32x16 oacc[NDB];
#pragma unroll
        for (int db = 0; db < NDB; ++db) oacc[db] = f32x16{};

        // Tile t+1's V and K rows are loaded into registers while tile t is
        // computed; at the top of each iteration they go to LDS (K and V
        // tiles shared by the four wavefronts).  Rows past the valid keys are
        // zeros.  Tile t+1's mask values are loaded as soon as tile t's
        // scores have taken theirs (one register set).
        u32x4 vreg[NVL], kreg[NVL];
        op_t mnext[2][2];     // additive mask values of the next tile
        uint64_t bnext[2][2];  // boolean mask bytes of the next tile
        const int nrec = key_lim > 0 ? int((int64_t(key_lim) * kvstride - int64_t(g) * D) * int64_t(sizeof(T))) : 0;
        const __amdgpu_buffer_rsrc_t krs =
            __builtin_amdgcn_make_buffer_rsrc(const_cast<T*>(kb), 0, nrec, 0x00020000);
        const __amdgpu_buffer_rsrc_t vrs =
            __builtin_amdgcn_make_buffer_rsrc(const_cast<T*>(vb), 0, nrec, 0x00020000);
        auto load_tile = [&](int t) __attribute__((always_inline)) {
            const int k0 = t * kMKeys;
#pragma unroll
            for (int i = 0; i < NVL; ++i) {
                // buffer loads over rows [0, key_lim) of this (batch, kv head):
                // rows past it, and head-dim chunks past D (given an offset
                // past the range), read as zeros without touching memory; no
                // branch, so every load is in flight together (byte offsets
                // fit 32 bits: S·Hkv·D·elt < 2^31 is checked on the host)
                const int ch = gtid + kMThreads * i, key = k0 + ch / CPR, col = 8 * (ch % CPR);
                const bool in_d = EXACT || col < D;
                const int boff = in_d ? int((int64_t(key) * kvstride + col) * int64_t(sizeof(T))) : 0x7ffffff0;
                vreg[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(vrs, boff, 0, 0));
                kreg[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(krs, boff, 0, 0));
            }
        };
        // mask values of keys k0 + 32·blk + 16·h + 8·gl + e (e < 8): the keys
        // of score registers 8h + e of block blk
        auto load_mask = [&](int t) __attribute__((always_inline)) {
            const int k0 = t * kMKeys;
            if constexpr (MASK) {
#pragma unroll
                for (int blk = 0; blk < 2; ++blk)
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        // addresses clamped into the row (keys at or past S are
                        // hidden anyway; with S a multiple of 8 a run of 8 is
                        // either inside or wholly past S); rows past S read
                        // row 0 of the plane (never written out)
                        const int key0 = k0 + 32 * blk + 16 * h + 8 * gl;
                        if constexpr (MK == 1) {
                            mnext[blk][h] = *reinterpret_cast<const op_t*>(mrow + (key0 + 8 <= S ? key0 : S - 8));
                        } else if constexpr (MK == 2) {
#pragma unroll
                            for (int e = 0; e < 8; ++e) mnext[blk][h][e] = mrow[key0 + e < S ? key0 + e : S - 1];
                        } else if constexpr (MK == 3) {
                            bnext[blk][h] = *reinterpret_cast<const uint64_t*>(mrow8 + (key0 + 8 <= S ? key0 : S - 8));
                        } else {
                            uint64_t w = 0;
#pragma unroll
                            for (int e = 0; e < 8; ++e)
                                w |= uint64_t(mrow8[key0 + e < S ? key0 + e : S - 1]) << (8 * e);
                            bnext[blk][h] = w;
                        }
                    }
            }
        };
        // this group's key tiles [tb, te); both groups run n_it iterations
        // (the same barriers), an iteration past the group's range idles
        const int t_mid = NG == 2 ? (ntile + 1) / 2 : ntile;
        const int tb = grp == 0 ? 0 : t_mid;
        const int te = grp == 0 ? t_mid : ntile;
        const int n_it = t_mid;
        // the staged registers (one tile's V and K rows) into LDS buffer buf
        auto write_tile = [&](int buf) __attribute__((always_inline)) {
            T* const vw = gbuf + buf * 2 * TILE;
#pragma unroll
            for (int i = 0; i < NVL; ++i) {
                const int ch = gtid + kMThreads * i;
                const int li = (ch / CPR) * ROWP + 8 * (ch % CPR);
                *reinterpret_cast<u32x4*>(vw + li) = vreg[i];
                *reinterpret_cast<u32x4*>(vw + TILE + li) = kreg[i];
            }
        };
        if (tb < te) {
            load_tile(tb);
            load_mask(tb);
        }
        if constexpr (NBUF == 2) {
            // tile tb into buffer 0 and tile tb+1's loads in flight; the
            // first barrier also covers the previous block's reads (and the
            // merge stash)
            __syncthreads();
            if (tb < te) {
                write_tile(0);
                if (tb + 1 < te) load_tile(tb + 1);
            }
            __syncthreads();
        }
        for (int it = 0; it < n_it; ++it) {
            const int t = tb + it;
            const bool active = t < te;  // uniform over the group
            const int k0 = t * kMKeys;
            const int cur = NBUF == 2 ? (it & 1) : 0;
            if constexpr (NBUF == 1) {
                __syncthreads();  // every wavefront is done reading the previous K and V tiles
                if (active) write_tile(0);
                __syncthreads();  // the tiles are in place
                if (!active) continue;
                if (t + 1 < te) load_tile(t + 1);
            } else {
                if (!active) {  // idle iteration: the same single barrier
                    __syncthreads();
                    continue;
                }
            }
            const T* const vt = gbuf + cur * 2 * TILE;
            const T* const kt = vt + TILE;

            // K operands from LDS: virtual row r of block blk is key 32·blk +
            // perm_row(r) of the tile, head dims 16c + 8gl .. +7
            const T* krow[2] = {kt + perm_row(r) * ROWP + 8 * gl, kt + (32 + perm_row(r)) * ROWP + 8 * gl};
            // Sᵀ = K·Qᵀ
            f32x16 sacc[2];
#pragma unroll
            for (int blk = 0; blk < 2; ++blk) {
                sacc[blk] = f32x16{};
#pragma unroll
                for (int c = 0; c < NC; ++c)
                    sacc[blk] = Op<T>::mma(*reinterpret_cast<const op_t*>(krow[blk] + 16 * c), qop[c], sacc[blk]);
            }
            // scaled scores plus mask, in log2 units; keys past S and (causal)
            // after the row are hidden
            float mt = -INFINITY;
#pragma unroll
            for (int blk = 0; blk < 2; ++blk)
#pragma unroll
                for (int f = 0; f < 16; ++f) {
                    const int key = k0 + 32 * blk + acc_pos(f, gl);
                    float sv = sacc[blk][f] * p.sl2;
                    if constexpr (MASK && !BMASK)
                        sv = fmaf(float(mnext[blk][(f >> 3) & 1][f & 7]), 1.44269504088896340736f, sv);
                    bool ok = key < key_lim && (!CAUSAL || key <= qrow);
                    if constexpr (BMASK) ok = ok && ((bnext[blk][(f >> 3) & 1] >> (8 * (f & 7))) & 0xff) != 0;
                    sv = ok ? sv : -INFINITY;
                    sacc[blk][f] = sv;
                    mt = fmaxf(mt, sv);
                }
            mt = fmaxf(mt, xor32(mt));
            if (MASK && t + 1 < te) load_mask(t + 1);  // this tile's mask values are used
            const float m_new = fmaxf(m_run, mt);
            const float alpha = m_new == -INFINITY ? 1.0f : __builtin_amdgcn_exp2f(m_run - m_new);
            const float mu = m_new == -INFINITY ? 0.0f : m_new;
            m_run = m_new;
            l_run *= alpha;
            l_ex *= alpha;
#pragma unroll
            for (int db = 0; db < NDB; ++db) oacc[db] *= alpha;
            op_t pop[2][2];  // P operand of block blk, 16-key step kc: registers 8kc .. 8kc+7
#pragma unroll
            for (int blk = 0; blk < 2; ++blk)
#pragma unroll
                for (int kc = 0; kc < 2; ++kc)
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const float pe = __builtin_amdgcn_exp2f(sacc[blk][8 * kc + e] - mu);
                        const T pr = static_cast<T>(pe);
                        l_ex += pe;
                        l_run += float(pr);
                        pop[blk][kc][e] = pr;
                    }
            // Oᵀ += Vᵀ·Pᵀ
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
                            half[h] = lds_read_tr16(vt + key * ROWP + 32 * db + tr_col);
                        }
                        const op_t va = __builtin_bit_cast(op_t, __builtin_shufflevector(half[0], half[1], 0, 1, 2, 3, 4, 5, 6, 7));
                        oacc[db] = Op<T>::mma(va, pop[blk][kc], oacc[db]);
                    }
            if constexpr (NBUF == 2) {
                // tile t+1 (its loads landed during this tile) into the other
                // buffer, tile t+2's loads in flight; one barrier publishes it
                // and retires this tile's reads of the current buffer
                if (t + 1 < te) {
                    write_tile(cur ^ 1);
                    if (t + 2 < te) load_tile(t + 2);
                }
                __syncthreads();
            }
        }

        // merge the two key halves: group 1 leaves (m, l, l_exact, Oᵀ) in LDS,
        // group 0 combines m = max(m0, m1), O = O0·2^(m0-m) + O1·2^(m1-m),
        // likewise the sums, and writes the block
        if constexpr (NG == 2) {
            __syncthreads();  // every tile read of this block is done
            float* stash = reinterpret_cast<float*>(lds);
            if (grp == 1) {
#pragma unroll
                for (int db = 0; db < NDB; ++db)
#pragma unroll
                    for (int f = 0; f < 16; ++f) stash[((w4 * NDB + db) * 16 + f) * 64 + lane] = oacc[db][f];
                s_ml[w4][0][lane] = m_run;
                s_ml[w4][1][lane] = l_run;
                s_ml[w4][2][lane] = l_ex;
            }
            __syncthreads();
            if (grp == 1) continue;
            const float m1 = s_ml[w4][0][lane];
            const float mm = fmaxf(m_run, m1);
            const float a0 = mm == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m_run - mm);
            const float a1 = mm == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m1 - mm);
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int f = 0; f < 16; ++f)
                    oacc[db][f] = oacc[db][f] * a0 + stash[((w4 * NDB + db) * 16 + f) * 64 + lane] * a1;
            l_run = l_run * a0 + s_ml[w4][1][lane] * a1;
            l_ex = l_ex * a0 + s_ml[w4][2][lane] * a1;
            m_run = mm;
        }

        // O = Oᵀ / l (the sum of the rounded probabilities, over both lane halves),
        // LSE from the exact sum; a row with no visible key writes zeros and -inf
        const float l_tot = l_run + xor32(l_run);
        const float l_e = l_ex + xor32(l_ex);
        if (live) {
            const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
            T* orow = static_cast<T*>(p.o) + (int64_t(b) * S + qrow) * qstride + int64_t(hq) * D;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    T vals[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) vals[e] = static_cast<T>(oacc[db][8 * h + e] * inv);
                    // head dims 32db + 16h + 8gl .. +7
                    if (32 * db + 16 * h + 8 * gl < D)
                        *reinterpret_cast<u32x4*>(orow + 32 * db + 16 * h + 8 * gl) =
                            *reinterpret_cast<const u32x4*>(vals);
                }
            if (p.lse && gl == 0)
                p.lse[(int64_t(b) * p.Hq + hq) * S + qrow] =
                    l_e > 0.0f ? (m_run + __builtin_amdgcn_logf(l_e)) * 0.69314718055994530942f : -INFINITY;
        }
    }
}

template <typename T, int DP, bool CAUSAL, int MK, bool EXACT>
int launch_m(const attn_detail::LaunchArgs& a) {
    MParams mp;
    mp.q = a.q;
    mp.k = a.k;
    mp.v = a.v;
    mp.mask = a.mask;
    mp.o = a.o;
    mp.lse = a.lse;
    mp.S = int(a.S);
    mp.Hq = int(a.Hq);
    mp.Hkv = int(a.Hkv);
    mp.group = int(a.Hq / a.Hkv);
    mp.D = int(a.D);
    mp.pad_lens = a.padded ? a.pad_lens : nullptr;
    mp.mask_b = a.mask_b;
    mp.mask_h = a.mask_h;
    mp.sl2 = a.scale * 1.44269504088896340736f;
    mp.n_qb = int((a.S + kMRows - 1) / kMRows);
    // Two-group workgroups (one per CU) always pair heavy and light causal
    // blocks.  One-group workgroups pair them only when the paired launch
    // still has two workgroups for each of the 256 CUs: below that, two
    // resident workgroups per CU hide more of the per-tile load latency than
    // the balance gains.
    constexpr int NG = MGroups<DP>::value;
    mp.pair = CAUSAL && (NG == 2 || int64_t((mp.n_qb + 1) / 2) * a.Hq * a.B >= 512) ? 1 : 0;
    const unsigned n_x = unsigned(mp.pair ? (mp.n_qb + 1) / 2 : mp.n_qb);
    attn_detail::log_launch("masked_kernel<%s, DP=%d, causal=%d, mask_mode=%d, exact=%d> groups=%d grid=(%u, %lld, %lld) "
                            "block=%d pair=%d D=%lld S=%lld",
                            attn_detail::dtype_name(a.dtype), DP, int(CAUSAL), MK, int(EXACT), NG, n_x, (long long)a.Hq,
                            (long long)a.B, kMThreads * NG, mp.pair, (long long)a.D, (long long)a.S);
    hipLaunchKernelGGL((masked_kernel<T, DP, CAUSAL, MK, EXACT>), dim3(n_x, unsigned(a.Hq), unsigned(a.B)),
                       dim3(kMThreads * NG), 0, static_cast<hipStream_t>(a.stream), mp);
    const hipError_t e = hipGetLastError();
    if (e == hipSuccess) return ATTN_OK;
    if (e == hipErrorNoBinaryForGpu || e == hipErrorInvalidDeviceFunction) return ATTN_ERR_DEVICE;
    return ATTN_ERR_LAUNCH;
}

template <typename T, int DP, int MK>
int launch_mc(const attn_detail::LaunchArgs& a) {
    if (a.D == DP)
        return a.causal ? launch_m<T, DP, true, MK, true>(a) : launch_m<T, DP, false, MK, true>(a);
    return a.causal ? launch_m<T, DP, true, MK, false>(a) : launch_m<T, DP, false, MK, false>(a);
}

template <typename T, int DP, bool MASK>
int launch_mk(const attn_detail::LaunchArgs& a) {
    if (!MASK) return launch_mc<T, DP, 0>(a);
    if (a.mask_bool) return a.S % 8 == 0 ? launch_mc<T, DP, 3>(a) : launch_mc<T, DP, 4>(a);
    return a.S % 8 == 0 ? launch_mc<T, DP, 1>(a) : launch_mc<T, DP, 2>(a);
}

// head dim padded to the next multiple of 32 (D is a multiple of 16 in [16, 256])
template <typename T, bool MASK>
int launch_mt(const attn_detail::LaunchArgs& a) {
    switch ((a.D + 31) / 32) {
        case 1: return launch_mk<T, 32, MASK>(a);
        case 2: return launch_mk<T, 64, MASK>(a);
        case 3: return launch_mk<T, 96, MASK>(a);
        case 4: return launch_mk<T, 128, MASK>(a);
        case 5: return launch_mk<T, 160, MASK>(a);
        case 6: return launch_mk<T, 192, MASK>(a);
        case 7: return launch_mk<T, 224, MASK>(a);
        default: return launch_mk<T, 256, MASK>(a);
    }
}

}  // namespace

namespace attn_detail {

int launch_masked(const LaunchArgs& a) {
    return a.dtype == ATTN_BF16 ? launch_mt<__bf16, true>(a) : launch_mt<_Float16, true>(a);
}

int launch_general(const LaunchArgs& a) {
    return a.dtype == ATTN_BF16 ? launch_mt<__bf16, false>(a) : launch_mt<_Float16, false>(a);
}

}  // namespace attn_detail
