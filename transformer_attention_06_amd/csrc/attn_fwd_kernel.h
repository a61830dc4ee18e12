// attn_fwd_kernel.h — the fused attention forward kernel template for gfx950
// (MI355X) and its launcher; instantiated per element type and head dim by
// attn_fwd_<type>_d<D>.hip, so the instances compile in parallel.  Internal
// to the library.
//
//
// A group of 4 wavefronts of 64 lanes owns one (batch, query head, 128-row
// query block); each wavefront owns 32 query rows.  A workgroup is one group,
// or two under causal masking with 16-bit inputs (a heavy and a light block
// of one head, see the work decomposition below).  K/V tiles of BN
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
#pragma once

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <type_traits>

#include "attn_fwd.h"
#include "attn_fwd_common.h"
#include "attn_launch.h"


namespace {


constexpr int kThreads = 256;
constexpr int BM = attn_detail::kBlockM;  // 128 query rows per workgroup
static_assert(BM == 4 * 32, "4 wavefronts x 32 rows");

// Wavefront groups per workgroup: two for the 16-bit types under causal
// masking (eight wavefronts, two per SIMD, a heavy and a light query block
// in one workgroup), otherwise one: without causal masking every block of a
// sequence costs the same, so independent 4-wave workgroups (two per CU)
// need no pairing and no shared barrier; fp32 registers do not fit twice per
// SIMD.
// Head dims above 160 (16-bit types) run one group with one wavefront per
// SIMD: their output accumulators (8 blocks at D = 256) live in AGPRs
// beside a full set of VGPRs.  At D = 64 (16-bit, one-group workgroups,
// no LSE, no mask tensor) a wavefront fits in 168 registers, without
// spills, with operands read three MFMAs ahead instead of six, so three
// workgroups share a CU (three wavefronts per SIMD): at this head dim the
// softmax's VALU stream outweighs the MFMAs, and a third wavefront fills
// more of its stalls.
template <typename T, int D, bool CAUSAL>
struct Groups {
    static constexpr int value = sizeof(T) == 2 && CAUSAL && D <= 160 ? 2 : 1;
};
template <typename T, int D, bool CAUSAL, bool LSE, int MK>
struct WavesPerSimd {
    static constexpr int value =
        sizeof(T) == 2 && D > 160 ? 1 : (sizeof(T) == 2 && D == 64 && !CAUSAL && !LSE && MK == 0 ? 3 : 2);
};

// Work of one group: one (batch, query head, 128-row query block); four
// wavefronts of 32 rows each.  Two groups share a CU (two wavefronts per
// SIMD; three at D = 64, see WavesPerSimd), so the stalls of one
// wavefront's stream are filled by the other's: one-group workgroups, or
// one workgroup of two groups pairing a causal heavy and light block.
//
// Each wavefront software-pipelines its own tile loop.  Step j (key tile j)
// is one fixed instruction stream of two parts:
//   A: the MFMAs of Sᵀ(j+1) = K(j+1)·Qᵀ, interleaved with the running-max
//      update and the first half of the exponentials of S(j);
//   B: the MFMAs of Oᵀ += Vᵀ(j)·Pᵀ(j), interleaved with the remaining
//      exponentials, packing P(j) into MFMA operands, the row sums, and the
//      mask and row maxima of S(j+1).
// MFMA operands are read from LDS PF products ahead of their use.  K and V
// tiles are double-buffered in LDS; step j loads K tile j+2 and V tile j+1
// (one 1 KiB direct load per wavefront every few MFMAs) and ends with a wait
// for those loads and one workgroup barrier.
// MK: 0 no mask tensor; 1 an additive mask tensor in T; 2 a boolean mask
// tensor (one byte per entry, nonzero: the key takes part).  With a mask
// tensor each wavefront stages the 32 x BN block of its own rows for the
// next tile in an LDS region of its own (direct loads at the start of the
// step, waited on by that wavefront alone), and adds it to (or selects)
// the scores of that tile before their row maxima are taken.
template <typename T, int D, bool CAUSAL, bool PAD, bool LSE, bool ROPE, int MK = 0>
__global__ __launch_bounds__(kThreads * (Groups<T, D, CAUSAL>::value), (WavesPerSimd<T, D, CAUSAL, LSE, MK>::value))
void attn_fwd_kernel(
    KParams p) {
    using E = Elem<T>;
    using op_t = typename E::op_t;
    constexpr int KPL = E::KPL;
    // 64-key tiles; 32 for the 16-bit head dims above 128, whose wider rows
    // and output accumulators leave room for half the score registers only
    constexpr int BN = sizeof(T) == 2 && D > 128 ? 32 : E::BN;
    constexpr int ES = int(sizeof(T));
    constexpr int CH = 16 / ES;            // elements per 16-byte slot
    // LDS tile rows hold DL head dims, D rounded up to a power of two: with
    // D < DL (80, 96, 112, 144, 160; 16-bit types) the 16-byte slots at or
    // past D are loaded as zeros and never read by a K operand; the O
    // blocks past D multiply zero V columns and are not stored
    constexpr int DL = D <= 64 ? 64 : D <= 128 ? 128 : 256;
    static_assert(D <= 256, "head dim");
    static_assert(D % 16 == 0 && D <= DL && (D == DL || sizeof(T) == 2), "head dim");
    constexpr int NS = DL / CH;            // slots per tile row
    constexpr int ROW_B = DL * ES;         // bytes per tile row
    constexpr int TILE_E = BN * DL;        // elements per K (or V) tile
    constexpr int NLD = BN * ROW_B / 4096; // 1 KiB direct loads per wave per tile
    static_assert(NLD * 4096 == BN * ROW_B, "tile split into 1 KiB wave loads");
    constexpr int NC = D / (2 * KPL);      // MFMA steps along D (Sᵀ)
    constexpr int NBLK = BN / 32;          // 32-key blocks per tile
    constexpr int NKC = BN / (2 * KPL);    // MFMA steps along keys (Oᵀ)
    constexpr int NDB = (D + 31) / 32;     // 32-dim blocks of O
    constexpr int NF = 16 * NBLK;          // scores per lane per tile
    constexpr int NG = Groups<T, D, CAUSAL>::value;  // wavefront groups
    constexpr int WPS = WavesPerSimd<T, D, CAUSAL, LSE, MK>::value;
    constexpr bool ACC_A = WPS == 1;       // output accumulators in AGPRs
    constexpr int NBUF = 2;                // LDS buffers per operand and group
    constexpr int KD = NBUF == 4 ? 3 : 2;  // step t loads K tile t+KD
    constexpr int VD = NBUF == 4 ? 3 : 1;  // and V tile t+VD
    constexpr int N1 = NC * NBLK;          // Sᵀ MFMAs per tile
    constexpr int N2 = NKC * NDB;          // P·V MFMAs per tile
    constexpr int PF = WPS == 3 ? 3 : 6;   // operand prefetch distance (MFMAs)
    static_assert(NBUF * TILE_E * ES <= 65536, "buffer offsets fit the LDS immediate");

    // Per group: K tiles [NBUF][BN][DL], then V tiles [NBUF][BN][DL], slots
    // swizzled.
    __shared__ __attribute__((aligned(1024))) T lds[NG * 2 * NBUF * TILE_E];
    // Mask tensor tiles: per wavefront 32 rows x BN entries in NML blocks of
    // 1 KiB, block i holding keys [MKPL·i, MKPL·(i+1)) of all 32 rows (32
    // bytes per row: two 16-byte chunks, swapped on rows 8..15 and 24..31
    // so that the 16 (32) lanes of one LDS read pass hit distinct banks).
    // Block i is one direct load, so the scores of key block i can be masked
    // as soon as that load has landed.
    static_assert(MK == 0 || sizeof(T) == 2, "mask tensors with 16-bit inputs only");
    constexpr int ME = MK == 1 ? int(sizeof(T)) : 1;  // bytes per mask entry
    constexpr int MWAVE_B = MK ? 32 * BN * ME : 0;    // one wavefront's rows of a tile
    constexpr int NML = MWAVE_B / 1024;               // 1 KiB loads per wavefront per tile
    constexpr int MKPL = 1024 / (32 * ME);            // keys per load
    static_assert(MK == 0 || (NML * 1024 == MWAVE_B && MKPL * ME == 32), "mask tile split into 1 KiB loads");
    __shared__ __attribute__((aligned(1024))) uint8_t mlds[MK ? NG * 4 * MWAVE_B : 16];

    // ---- work decomposition ------------------------------------------------
    // Workgroup i runs on XCD i % 8.  Logical units (batch, kv head, query
    // head) are split into 8 contiguous ranges, one per XCD, so the query
    // heads sharing a K/V head share that XCD's L2.  Without causal masking
    // the query blocks of a unit are dispatched one after another (task-minor
    // order): they all stream the same K/V tiles from the first, at about the
    // same time, so the tiles are read from memory once and shared in L2.
    const int wg = blockIdx.x;
    int unit, task;
    if (p.xcd_chunk > 0 && !CAUSAL) {
        const int xcd = wg & 7, local = wg >> 3;
        task = local % p.n_qb;
        unit = xcd * p.xcd_chunk + local / p.n_qb;
    } else if (p.xcd_chunk > 0) {
        const int xcd = wg & 7, local = wg >> 3;
        task = local / p.xcd_chunk;
        unit = xcd * p.xcd_chunk + local % p.xcd_chunk;
    } else {
        task = wg / p.n_units;
        unit = wg % p.n_units;
    }
    const int jg = unit % p.group;
    const int bg = unit / p.group;
    const int g = bg % p.Hkv;
    const int b = bg / p.Hkv;
    const int hq = g * p.group + jg;

    // Rows of this batch entry: with packed sequences (offsets cu[0..B]),
    // sequence b is rows [cu[b], cu[b+1]) of one (1, T, H, D) buffer, and its
    // length replaces S.  The offsets are clamped into [0, T] and the length
    // to the launch's maximum (p.S), so every access stays inside the buffers
    // whatever the offsets hold.
    int S = p.S;
    int64_t row0 = 0;  // first row of this batch entry's sequence
    if (p.cu) {
        int s0 = p.cu[b], s1 = p.cu[b + 1];
        s0 = s0 < 0 ? 0 : (s0 > p.total ? p.total : s0);
        s1 = s1 < s0 ? s0 : (s1 > p.total ? p.total : s1);
        S = s1 - s0 < p.S ? s1 - s0 : p.S;
        row0 = s0;
    }
    const int n_qb = p.cu ? (S + BM - 1) / BM : p.n_qb;

    // With two groups (causal masking only) a task is a pair of query blocks
    // of one (batch, query head): the heaviest and the lightest remaining
    // block (qh = n_qb-1-task, ql = task).  Group 0 takes the heavy block's
    // key tiles up to its last nb, group 1 the light block and then those
    // last nb tiles; nb evens out the two groups' tile counts, and the heavy
    // block's two partial softmax states are merged through LDS at the end.
    // With one group a task is one block; under causal masking heaviest
    // first for the first half of the launch and lightest first for the
    // second half (two workgroups per CU even out).  A packed sequence
    // shorter than the longest has fewer blocks: its surplus tasks leave here,
    // before any barrier (the whole workgroup shares b and task).
    int qh = task, ql = -1;
    if (NG == 2) {
        static_assert(!(NG == 2 && !CAUSAL), "two groups only pair causal blocks");
        qh = n_qb - 1 - task;
        ql = task < qh ? task : -1;
        if (task > qh) return;
    } else {
        if (task >= n_qb) return;
        if (CAUSAL) {
            const int half = (n_qb + 1) >> 1;
            qh = task < half ? n_qb - 1 - task : task - half;
        }
    }

    int key_lim = S;
    if (PAD) {
        const int L = p.pad_lens[b];
        key_lim = L < 0 ? 0 : (L > S ? S : L);
    }
    // key tiles with at least one visible key for query block q
    auto tiles_of = [&](int q) __attribute__((always_inline)) {
        if (q < 0) return 0;
        int e = key_lim;
        if (CAUSAL) e = e < q * BM + BM ? e : q * BM + BM;
        return (e + BN - 1) / BN;
    };
    const int Th = tiles_of(qh);
    const int Tl = tiles_of(ql);
    int nb = 0;
    // Both groups pass the same barriers, one per step, so the work is
    // balanced by barrier count: group 0 (the heavy block's first Th - nb
    // tiles) passes Th - nb + 1, group 1 (light block, then the heavy block's
    // last nb tiles, one barrier between) Tl + nb + 3.
    if (NG == 2) nb = ql >= 0 ? (Th - Tl > 2 ? (Th - Tl - 2) / 2 : 0) : Th / 2;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    // wavefront index, made provably uniform so branches on it are scalar
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int w4 = wave & 3;
    const int grp = NG == 2 ? (wave >> 2) : 0;
    T* const lds_k = lds + grp * 2 * NBUF * TILE_E;
    T* const lds_v = lds_k + NBUF * TILE_E;

    // this group's segments: (query block, key tiles [t0, t1), written out
    // at its end or kept for the merge)
    int nseg = 0, seg_q0 = 0, seg_a0 = 0, seg_b0 = 0, seg_q1 = 0, seg_a1 = 0, seg_b1 = 0;
    bool seg_out0 = true, seg_out1 = true;
    auto add_seg = [&](int q, int a, int e, bool out) __attribute__((always_inline)) {
        if (nseg == 0) {
            seg_q0 = q, seg_a0 = a, seg_b0 = e, seg_out0 = out;
        } else {
            seg_q1 = q, seg_a1 = a, seg_b1 = e, seg_out1 = out;
        }
        ++nseg;
    };
    // group 0 starts at the heavy block's first key tile, as group 1 starts
    // at the light block's: every group of a head streams from tile 0 at the
    // start of the launch, so the workgroups of a head read the same tiles at
    // about the same time (L2 hits) instead of each from its own split point
    if (grp == 0) {
        add_seg(qh, 0, Th - nb, nb == 0);
    } else {
        if (ql >= 0) add_seg(ql, 0, Tl, true);
        if (nb > 0) add_seg(qh, Th - nb, Th, false);
    }
    // barriers a segment of n tiles passes (initial loads, Sᵀ of its first
    // tile, one per further tile); the groups pad to the same total
    auto seg_bars = [](int n) { return n > 0 ? n + 1 : 0; };
    const int bars0 = seg_bars(Th - nb);
    const int bars1 = (ql >= 0 ? seg_bars(Tl) : 0) + (nb > 0 ? seg_bars(nb) : 0) + (ql >= 0 && nb > 0 ? 1 : 0);
    const int bars_all = NG == 2 ? (bars0 > bars1 ? bars0 : bars1) : bars0;
    int n_bar = 0;
    int seg_end = 0;  // key tiles at or past this index are not loaded
    const int r = lane & 31;
    const int gl = lane >> 5;

    const int64_t qstride = int64_t(p.Hq) * D;
    const int64_t kvstride = int64_t(p.Hkv) * D;
    // element offsets of this batch entry's first row in q / out and in k, v
    const int64_t q_off = p.cu ? row0 * qstride : int64_t(b) * p.q_bstride;
    const int64_t kv_off = p.cu ? row0 * kvstride : int64_t(b) * p.kv_bstride;
    const T* qbase = static_cast<const T*>(p.q) + q_off + int64_t(hq) * D;
    const T* kbase = static_cast<const T*>(p.k) + kv_off + int64_t(g) * D;
    const T* vbase = static_cast<const T*>(p.v) + kv_off + int64_t(g) * D;

    // ---- tile loads: global -> LDS directly -------------------------------
    // Buffer resources cover this (batch, kv head) slice; rows at or past S
    // read as zero.  Wave w fills bytes [w·NLD KiB, (w+1)·NLD KiB) of each
    // tile; lane l writes the 16-byte slot at l·16 of its KiB, i.e. row
    // (KiB offset + 16 l) / ROW_B at physical slot p, which holds logical slot
    // p ^ swz(row) of that key row.  A tile past the last one is "loaded" with
    // an empty resource (every lane out of range), so every step issues the
    // same loads and waits on the same count.
    const uint32_t kv_bytes = uint32_t((int64_t(S) * kvstride - int64_t(g) * D) * int64_t(ES));
    const i32x4 krs = rsrc_words(kbase, kv_bytes);
    const i32x4 vrs = rsrc_words(vbase, kv_bytes);
    const i32x4 krs0 = rsrc_words(kbase, 0);
    const i32x4 vrs0 = rsrc_words(vbase, 0);
    const uint32_t row_bytes = uint32_t(kvstride * int64_t(ES));
    // Load i of a wave covers tile rows rw_i + [0, RPL) with rw_i =
    // (w·NLD + i)·RPL; lane l takes row rw_i + lr, physical slot ps.  The
    // swizzle is a bit permutation of the row index and rw_i shares no bits
    // with lr, so the logical slot is ps ^ swz(lr) ^ swz(rw_i): one per-lane
    // offset, XORed with a uniform term per load.
    constexpr int RPL = 1024 / ROW_B;  // tile rows per 1 KiB load
    const int lr = lane / (ROW_B / 16);
    const int ps = lane % (ROW_B / 16);
    const uint32_t ld_base = uint32_t(lr) * row_bytes + uint32_t((ps ^ swz<NS>(lr)) * 16);
    // With D < DL the offsets are formed once per load index instead (the
    // row stride need not be a multiple of the row's 2^k bytes, so the XOR
    // cannot act on the whole offset), and the padding slots point past the
    // buffer's end: they read as zero.
    uint32_t ld_off[D < DL ? NLD : 1];
    if constexpr (D < DL) {
#pragma unroll
        for (int i = 0; i < NLD; ++i) {
            const int rw = (w4 * NLD + i) * RPL;
            const int ls = ps ^ swz<NS>(lr) ^ swz<NS>(rw);
            ld_off[i] = ls < D / CH ? uint32_t(rw + lr) * row_bytes + uint32_t(ls * 16) : 0x80000000u;
        }
    }
    const uint32_t lds_k_b = uint32_t(reinterpret_cast<uintptr_t>(lds_k));
    const uint32_t lds_v_b = uint32_t(reinterpret_cast<uintptr_t>(lds_v));
    // Buffer resource of one key tile: the slice from key row t·BN on, empty
    // for a tile at or past the segment end (every lane then out of range, so
    // the load writes zeros and reads no memory).  All scalar.
    const uint64_t kaddr = reinterpret_cast<uint64_t>(kbase);
    const uint64_t vaddr = reinterpret_cast<uint64_t>(vbase);
    auto tile_rsrc = [&](uint64_t base, int t) __attribute__((always_inline)) {
        const uint32_t off = uint32_t(t * BN) * row_bytes;
        const bool live = t < seg_end && off < kv_bytes;
        const uint64_t a = base + off;
        return i32x4{__builtin_amdgcn_readfirstlane(int(uint32_t(a))),
                     __builtin_amdgcn_readfirstlane(int(uint32_t(a >> 32) & 0xffff)),
                     __builtin_amdgcn_readfirstlane(int(live ? kv_bytes - off : 0u)), 0x00020000};
    };
    const uint32_t lds_k_s = __builtin_amdgcn_readfirstlane(lds_k_b);
    const uint32_t lds_v_s = __builtin_amdgcn_readfirstlane(lds_v_b);
    // load li (0..NLD-1) of a tile with resource rs into LDS buffer buf
    auto load_part = [&](const i32x4& rs, uint32_t lds_s, int buf, int li) __attribute__((always_inline)) {
        uint32_t voff;
        if constexpr (D < DL) {
            voff = ld_off[li];
        } else {
            const int rw = (w4 * NLD + li) * RPL;
            uint32_t lb = ld_base;
            asm volatile("" : "+v"(lb));  // formed here, not hoisted as one register per load
            voff = (lb ^ uint32_t(swz<NS>(rw) * 16)) + uint32_t(rw) * row_bytes;
        }
        lds_dma16(rs, lds_s + uint32_t(buf * TILE_E * ES) + uint32_t((w4 * NLD + li) * 1024), voff);
    };
    // load i (0..2·NLD-1): K tile tk into K buffer kbuf for i < NLD, else V
    // tile tv into V buffer vbuf.  Buffers are counted from the segment's
    // first tile, so that inside the two-step loop body they are constants.
    auto load_one = [&](int tk, int tv, int kbuf, int vbuf, int i) __attribute__((always_inline)) {
        if (i < NLD)
            load_part(tile_rsrc(kaddr, tk), lds_k_s, kbuf, i);
        else
            load_part(tile_rsrc(vaddr, tv), lds_v_s, vbuf, i - NLD);
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
    // the constant 16·kc·DL
    int v_off[NDB][2];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int key = 8 * gl + 4 * h + tr_key;
            const int col = 32 * db + tr_col;
            v_off[db][h] = key * DL + (((col / CH) ^ swz<NS>(key)) * CH) + col % CH;
        }
    const float sl2 = p.sl2;

    // ---- this wave's 32 rows of the current segment's block ----------------
    int wrow0 = 0, qrow = 0;
    op_t qv[NC];
    f32x16 oacc[NDB];
    float m_run = -INFINITY;  // running max (scaled, log2)
    float l_run = 0.0f;       // sum of the rounded probabilities
    float l_lse = 0.0f;       // sum of the exact probabilities (LSE)
    auto begin_rows = [&](int q) __attribute__((always_inline)) {
        wrow0 = q * BM + w4 * 32;
        qrow = wrow0 + r;
        if (qrow < S) {
            const T* qr = qbase + int64_t(qrow) * qstride;
#pragma unroll
            for (int c = 0; c < NC; ++c) qv[c] = load_op<op_t>(qr + c * 2 * KPL + gl * KPL);
        } else {
#pragma unroll
            for (int c = 0; c < NC; ++c) qv[c] = op_t{};
        }
        if constexpr (ROPE) {
            // Rotary embedding of the Q tile in registers ([ATB-guide] §4.1
            // fifth fusion pattern, §8.4): pair (2i, 2i+1) turns by the row's
            // position × theta_i; the rotated values are rounded to T, as the
            // MFMA operand.
            const int pos = qrow < S ? (p.rope_pos ? p.rope_pos[int64_t(b) * S + qrow] : qrow) : 0;
            // theta_i = rho^i with rho = base^(-2/D) (from the host), read
            // through an opaque copy so that nothing stays live across the
            // tile loop
            double r1 = p.rope_r1;
            asm volatile("" : "+v"(r1));
            const double r4 = (r1 * r1) * (r1 * r1);
            const double r8 = r4 * r4;
            if constexpr (KPL == 1) {
                // lane gl holds dimension 2c + gl: the pair's other half sits
                // in the lane 32 away
                // theta_i / 2pi = rho^i / 2pi, stepped by multiplication
                double f = 0.15915494309189533577;
#pragma unroll
                for (int c = 0; c < NC; ++c) {
                    asm volatile("" : "+v"(f));  // one pair at a time: bounded registers
                    float cs, sn;
                    rope_cs<T>(pos, f, cs, sn);
                    f *= r1;
                    const float mine = qv[c];
                    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mine), __float_as_uint(mine),
                                                                     false, false);
                    const float other = __uint_as_float(gl == 0 ? sw[1] : sw[0]);
                    qv[c] = gl == 0 ? mine * cs - other * sn : mine * cs + other * sn;
                }
            } else {
                // lane holds dimensions 16c + 8gl + 0..7: pairs 8c + 4gl + 0..3;
                // theta_i / 2pi = rho^i / 2pi, stepped by multiplication
                double fc = gl ? 0.15915494309189533577 * r4 : 0.15915494309189533577;
#pragma unroll
                for (int c = 0; c < NC; ++c) {
                    double f = fc;
#pragma unroll
                    for (int j = 0; j < KPL / 2; ++j) {
                        asm volatile("" : "+v"(f));  // one pair at a time: bounded registers
                        float cs, sn;
                        rope_cs<T>(pos, f, cs, sn);
                        const float x0 = float(qv[c][2 * j]), x1 = float(qv[c][2 * j + 1]);
                        qv[c][2 * j] = to_t<T>(x0 * cs - x1 * sn);
                        qv[c][2 * j + 1] = to_t<T>(x1 * cs + x0 * sn);
                        f *= r1;
                    }
                    fc *= r8;
                }
            }
        }
        if constexpr (ACC_A) {
#pragma unroll
            for (int c = 0; c < NC; ++c) to_agpr(qv[c]);
        }
#pragma unroll
        for (int db = 0; db < NDB; ++db) oacc[db] = f32x16{};
        m_run = -INFINITY;
        l_run = 0.0f;
        l_lse = 0.0f;
    };

    // normalise and store O (and LSE) for this wave's rows
    auto write_rows = [&]() __attribute__((always_inline)) {
        const float l_tot = sum_xor32(l_run);
        const float l_e = LSE ? sum_xor32(l_lse) : 0.0f;
        const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
        if (qrow < S) {
            T* orow = static_cast<T*>(p.o) + q_off + int64_t(qrow) * qstride + int64_t(hq) * D;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    if (32 * db + 16 * h >= D) continue;  // padding dims (D % 16 == 0)
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
                // (B, Hq, S); packed sequences: (Hq, T)
                const int64_t li = p.cu ? int64_t(hq) * p.total + row0 + qrow : (int64_t(b) * p.Hq + hq) * S + qrow;
                p.lse[li] = lse;
            }
        }
    };

    // ---- MFMA operands from LDS ----------------------------------------------
    // Sᵀ product i (0..N1-1) of a K tile: head-dim step c = i / NBLK, key block
    // blk = i % NBLK
    auto fetch_k = [&](const T* ks, int i) __attribute__((always_inline)) -> op_t {
        const int c = i / NBLK, blk = i % NBLK;
        const int col = c * 2 * KPL + gl * KPL;
        const int off = (((col / CH) ^ xk) * CH) + col % CH;
        return load_op<op_t>(ks + (prow + 32 * blk) * DL + off);
    };
    // P·V product i (0..N2-1) of a V tile: key step kc = i / NDB, dim block db
    auto fetch_v = [&](const T* vs, int i) __attribute__((always_inline)) -> op_t {
        const int kcol = i / NDB, db = i % NDB;
        if constexpr (KPL == 1) {
            const int key = kidx(kcol, gl);
            const int col = 32 * db + prow;
            return vs[key * DL + (((col / CH) ^ swz<NS>(key)) * CH) + col % CH];
        } else {
            s16x4 half[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) half[h] = lds_read_tr16(vs + 16 * kcol * DL + v_off[db][h]);
            return __builtin_bit_cast(op_t, __builtin_shufflevector(half[0], half[1], 0, 1, 2, 3, 4, 5, 6, 7));
        }
    };

    // ---- softmax pieces ------------------------------------------------------
    // keys past the valid length, and keys after the row (causal), score -inf
    auto mask_tile = [&](f32x16 (&s)[NBLK], int t) __attribute__((always_inline)) {
        const int kb = t * BN;
        if ((kb + BN > key_lim) || (CAUSAL && kb + BN - 1 > wrow0)) {
            // key of register f = kb + 8·gl + kidx(f, 0); it is allowed below
            // lim = min(key_lim, qrow + 1): one compare per score against a
            // per-lane bound
            const int lim = CAUSAL ? (key_lim < qrow + 1 ? key_lim : qrow + 1) : key_lim;
            const int rel = lim - kb - 8 * gl;
#pragma unroll
            for (int blk = 0; blk < NBLK; ++blk)
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    if (kidx(16 * blk + i, 0) >= rel) s[blk][i] = -INFINITY;
        }
    };
    // ---- mask tensor tiles (MK != 0) ------------------------------------------
    // Plane (b', h') of the mask; a wavefront's block of tile t covers query
    // rows wrow0 + [0, 32) and keys t·BN + [0, BN).  Its loads read through
    // a buffer resource that ends at the end of the plane (rows past S read
    // as zero; keys past S within a row are hidden by mask_tile anyway).
    // The plane holds fewer than 2^31 bytes (checked on the host).
    const uint64_t mplane = MK ? reinterpret_cast<uint64_t>(p.mask) +
                                     (uint64_t(p.mask_b ? b : 0) * uint64_t(p.mask_h ? p.Hq : 1) +
                                      uint64_t(p.mask_h ? hq : 0)) * uint64_t(S) * uint64_t(S) * uint64_t(ME)
                               : 0;
    const uint32_t mplane_b = MK ? uint32_t(S) * uint32_t(S) * uint32_t(ME) : 0;
    const uint32_t mlds_w = __builtin_amdgcn_readfirstlane(
        uint32_t(reinterpret_cast<uintptr_t>(mlds)) + uint32_t(wave * MWAVE_B));
    const uint8_t* const mrow = mlds + wave * MWAVE_B + r * 32;  // this lane's row in block 0
    const int mhalf = (r >> 3) & 1;                                 // chunk swap of this lane's row
    // the wavefront's block of mask tile t into its region: lane l of load i
    // fills row l / 2, physical chunk l % 2
    auto load_mask = [&](int t) __attribute__((always_inline)) {
        if constexpr (MK != 0) {
            const uint32_t off = (uint32_t(wrow0) * uint32_t(S) + uint32_t(t * BN)) * uint32_t(ME);
            const uint64_t a = mplane + off;
            const i32x4 rs{__builtin_amdgcn_readfirstlane(int(uint32_t(a))),
                           __builtin_amdgcn_readfirstlane(int(uint32_t(a >> 32) & 0xffff)),
                           __builtin_amdgcn_readfirstlane(int(off < mplane_b ? mplane_b - off : 0u)), 0x00020000};
            const int row = lane >> 1;
            const uint32_t voff = uint32_t(row) * uint32_t(S * ME) + uint32_t(((lane & 1) ^ ((row >> 3) & 1)) * 16);
#pragma unroll
            for (int i = 0; i < NML; ++i)
                lds_dma16(rs, mlds_w + uint32_t(i * 1024), voff + uint32_t(i * MKPL * ME));
        }
    };
    // the load that brings the entries of scores 8j..8j+7 (keys 16j + 8·gl
    // + 0..7 of the lane's row), and those entries: 8 additive values (16
    // bytes) or 8 bytes
    auto mask_load_of = [](int j) __attribute__((always_inline)) { return 16 * j / MKPL; };
    using mchunk_t = typename std::conditional<MK == 2, uint2, u32x4>::type;
    auto read_mask = [&](int j) __attribute__((always_inline)) -> mchunk_t {
        const uint8_t* blk = mrow + mask_load_of(j) * 1024;
        if constexpr (MK == 2)
            return *reinterpret_cast<const uint2*>(blk + (((j & 1) ^ mhalf) * 16) + 8 * gl);
        else
            return *reinterpret_cast<const u32x4*>(blk + ((gl ^ mhalf) * 16));
    };
    // scores f = 8j + [e0, e1) of s take their mask entries from chunk m
    const float inv_scale = p.inv_scale;
    auto apply_mask = [&](f32x16 (&s)[NBLK], const mchunk_t& m, int j, int e0, int e1)
                          __attribute__((always_inline)) {
        if constexpr (MK != 0) {
#pragma unroll
            for (int e = e0; e < e1; ++e) {
                const int f = 8 * j + e;
                const float x = s[f >> 4][f & 15];
                if constexpr (MK == 2) {
                    const uint32_t w = e < 4 ? m.x : m.y;
                    s[f >> 4][f & 15] = ((w >> (8 * (e & 3))) & 0xffu) ? x : -INFINITY;
                } else {
                    const uint32_t w = m[e >> 1];
                    const uint16_t h = uint16_t(e & 1 ? w >> 16 : w);
                    s[f >> 4][f & 15] = fmaf(float(__builtin_bit_cast(T, h)), inv_scale, x);
                }
            }
        }
    };

    // Softmax work of one tile, split so it can ride along MFMAs:
    //   max_item(k): partial row maxima over scores 4k..4k+3 (four chains);
    //   fin0: the row max over both lane halves, scaled to log2 units;
    //   fin: running-max update (raised only when some row of the wave needs
    //        it: the exponentials then stay below 2^8 and the output needs no
    //        rescale), correction factor, scaling of the running sums;
    //   exp_item(f): the exponential of score f.
    constexpr int NMX = NF / 4;
    float mp[4];
    float mxs = -INFINITY;  // scaled row max of the tile whose maxima were taken last
    float pf[NF];
    float alpha = 1.0f, m_use = 0.0f;
    bool resc = false;
    auto max_item = [&](const f32x16 (&s)[NBLK], int k) __attribute__((always_inline)) {
        if (k < 4) mp[k] = -INFINITY;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int f = 4 * k + e;
            mp[k & 3] = fmaxf(mp[k & 3], s[f >> 4][f & 15]);
        }
        keep(mp[k & 3]);
    };
    auto fin0 = [&]() __attribute__((always_inline)) {
        const float mx = fmaxf(fmaxf(mp[0], mp[1]), fmaxf(mp[2], mp[3]));
        mxs = max_xor32(mx) * sl2;
        keep(mxs);
    };
    auto fin = [&]() __attribute__((always_inline)) {
        resc = __builtin_amdgcn_ballot_w64(mxs > m_run + kRescaleLog2) != 0;
        const float m_new = resc ? fmaxf(m_run, mxs) : m_run;
        alpha = (resc && m_new != -INFINITY) ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;
        l_run *= alpha;
        if constexpr (LSE) l_lse *= alpha;
        m_run = m_new;
        m_use = m_run == -INFINITY ? 0.0f : m_run;
        keep(m_use);
        keep(alpha);
    };
    auto exp_item = [&](const f32x16 (&s)[NBLK], int f) __attribute__((always_inline)) {
        touch(m_use);
        pf[f] = __builtin_amdgcn_exp2f(fmaf(s[f >> 4][f & 15], sl2, -m_use));
        keep(pf[f]);
    };
    // P operand kc from the exponentials, and its row sums
    float rs[2] = {0.0f, 0.0f}, rl[2] = {0.0f, 0.0f};
    auto pack_p = [&](const f32x16 (&s)[NBLK], op_t (&pb)[NKC], int kc) __attribute__((always_inline)) {
        if constexpr (KPL == 1) {
            float pv = pf[kc];
            pb[kc] = pv;
            rs[kc & 1] += pv;
            keep(rs[kc & 1]);
            keep(pb[kc]);
        } else {
            float x[KPL];
#pragma unroll
            for (int e = 0; e < KPL; ++e) {
                x[e] = pf[kc * KPL + e];
            }
#pragma unroll
            for (int e = 0; e < KPL; ++e) pb[kc][e] = to_t<T>(x[e]);
            typedef T t2 __attribute__((ext_vector_type(2)));
#pragma unroll
            for (int e = 0; e < KPL; e += 2) rs[(e >> 1) & 1] = sum2(t2{pb[kc][e], pb[kc][e + 1]}, rs[(e >> 1) & 1]);
            if constexpr (LSE) {
#pragma unroll
                for (int e = 0; e < KPL; ++e) rl[e & 1] += x[e];
                keep(rl[0]);
                keep(rl[1]);
            }
            keep(rs[0]);
            keep(rs[1]);
            asm volatile("" : : "v"(pb[kc]));  // packed here, before the wait states that follow
        }
    };
    auto finish_sums = [&]() __attribute__((always_inline)) {
        l_run += rs[0] + rs[1];
        if constexpr (LSE) l_lse += KPL == 1 ? rs[0] + rs[1] : rl[0] + rl[1];
        rs[0] = rs[1] = rl[0] = rl[1] = 0.0f;
    };
    auto rescale_o = [&]() __attribute__((always_inline)) {
        if (resc) {
#pragma unroll
            for (int db = 0; db < NDB; ++db) oacc[db] *= alpha;
        }
    };

    // ---- one pipelined step --------------------------------------------------
    // Tile t: S(t) arrives in sc, already masked and with its row maxima
    // taken (fin0 done); with G1, Sᵀ(t+1) is computed into sn from K buffer
    // 1 - par.  One operand stream covers both parts: K operands
    // 0..N1-1, then V operands 0..N2-1, each read PF MFMAs ahead (the first V
    // operands while part A still runs).
    //   part A: Sᵀ(t+1) MFMAs; the running-max update, then the exponentials
    //           of the first NKA P operands; loads of K tile t+2 and V
    //           tile t+1;
    //   part B: P(t)·V(t) MFMAs; the exponentials of the other P operands,
    //           each finished NDB MFMAs before its first use; the mask and
    //           row maxima of S(t+1).
    constexpr int NKA = (NKC + 1) / 2;     // P operands exponentiated in part A
    constexpr int NEA = NKA * KPL;         // their scores
    constexpr int MX0 = N2 / 8 > 1 ? N2 / 8 : 1;  // first part-B slot reading S(t+1)
    // part-B slot that takes row-max item k of S(t+1)
    constexpr auto mx_slot = [](int k) {
        for (int i = MX0; i < N2; ++i)
            if (k < (i - MX0 + 1) * NMX / (N2 - MX0)) return i;
        return N2 - 1;
    };
    // mask tensor: the part-B slot that reads the entries of scores 8j..8j+7
    // (two slots before their first row-max item), after waiting for the
    // load that brought them; the NML mask loads of a step precede its 2·NLD
    // tile loads, so load i has landed at vmcnt(2·NLD + NML - 1 - i)
    constexpr auto mrd_slot = [mx_slot](int j) { return mx_slot(2 * j) >= 2 ? mx_slot(2 * j) - 2 : 0; };
    auto mask_wait = [](int li) __attribute__((always_inline)) { wait_vmcnt(2 * NLD + NML - 1 - li); };
    mchunk_t mk[2];
    op_t pb[NKC];
    // par: (t - first tile of the segment) % 2; K tile t+1 is in K buffer
    // 1 - par, V tile t in V buffer par, and this step loads K tile t+2 into
    // K buffer par and V tile t+1 into V buffer 1 - par.
    auto step = [&](const int t, const int par, f32x16 (&sc)[NBLK], f32x16 (&sn)[NBLK],
                    const bool G1) __attribute__((always_inline)) {
        const T* kn = lds_k + (1 - par) * TILE_E;
        const T* vc = lds_v + par * TILE_E;
        constexpr int NL = 2 * NLD;  // tile loads of a step, spread over part A
        static_assert(NL <= N1, "one part-A slot per tile load at most");
        op_t fr[PF + 1];
        auto fetch = [&](int g) __attribute__((always_inline)) {
            fr[g % (PF + 1)] = g < N1 ? fetch_k(kn, g) : fetch_v(vc, g - N1);
        };
        const int g0 = G1 ? 0 : N1;  // first operand of this step
#pragma unroll
        for (int g = 0; g < PF; ++g)
            if (g0 + g < N1 + N2) fetch(g0 + g);
        // part A
#pragma unroll
        for (int i = 0; i < N1; ++i) {
            if (G1) {
                if (MK != 0 && i == 0) load_mask(t + 1);
#pragma unroll
                for (int k = 0; k < NL; ++k)
                    if (i == k * N1 / NL) load_one(t + KD, t + VD, par, 1 - par, k);
                if (i + PF < N1 + N2) fetch(i + PF);
                if constexpr (ACC_A) {
                    if (i < NBLK)
                        mfma_zero_qa(sn[i % NBLK], fr[i % (PF + 1)], qv[i / NBLK]);
                    else
                        mfma_acc_qa(sn[i % NBLK], fr[i % (PF + 1)], qv[i / NBLK]);
                } else {
                    if (i < NBLK)
                        mfma_zero(sn[i % NBLK], fr[i % (PF + 1)], qv[i / NBLK]);
                    else
                        mfma_acc(sn[i % NBLK], fr[i % (PF + 1)], qv[i / NBLK]);
                }
            }
            if (i == 0) fin();
            if (i > 0) {
#pragma unroll
                for (int f = (i - 1) * NEA / (N1 - 1); f < i * NEA / (N1 - 1); ++f) exp_item(sc, f);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int kc = 0; kc < NKA; ++kc) pack_p(sc, pb, kc);
        rescale_o();
        asm volatile("s_nop 4");  // VALU-written operands read by the next MFMA
        // part B
#pragma unroll
        for (int i = 0; i < N2; ++i) {
            if (N1 + i + PF < N1 + N2) fetch(N1 + i + PF);
            if constexpr (ACC_A)
                mfma_acc_a(oacc[i % NDB], fr[(N1 + i) % (PF + 1)], pb[i / NDB]);
            else
                mfma_acc(oacc[i % NDB], fr[(N1 + i) % (PF + 1)], pb[i / NDB]);
            // P operand kc (kc >= NKA) is formed over slots [(kc-1)·NDB, kc·NDB)
            if (i / NDB + 1 >= NKA && i / NDB + 1 < NKC) {
                const int kc = i / NDB + 1, j = i % NDB;
#pragma unroll
                for (int e = j * KPL / NDB; e < (j + 1) * KPL / NDB; ++e) exp_item(sc, kc * KPL + e);
                if (j == NDB - 1) {
                    pack_p(sc, pb, kc);
                    asm volatile("s_nop 1");  // read by the next MFMA
                }
            }
            if (G1) {
                if constexpr (MK != 0) {
#pragma unroll
                    for (int mj = 0; mj < NF / 8; ++mj)
                        if (i == mrd_slot(mj)) {
                            mask_wait(mask_load_of(mj));
                            mk[mj & 1] = read_mask(mj);
                        }
                }
                if (i == MX0) mask_tile(sn, t + 1);
                if (i >= MX0) {
#pragma unroll
                    for (int k = (i - MX0) * NMX / (N2 - MX0); k < (i - MX0 + 1) * NMX / (N2 - MX0); ++k) {
                        apply_mask(sn, mk[(k >> 1) & 1], k >> 1, 4 * (k & 1), 4 * (k & 1) + 4);
                        max_item(sn, k);
                    }
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        finish_sums();
        if (G1) fin0();
    };
    // wait for this wave's loads of the previous step, then publish
    auto end_step = [&]() __attribute__((always_inline)) {
        static_assert(2 * NLD < 16, "vmcnt immediate");
        if constexpr (NBUF == 4)
            __builtin_amdgcn_s_waitcnt(0x0F70 | (2 * NLD));  // vmcnt(2·NLD): the loads of step t-1 landed
        else
            __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this step's loads landed
        __syncthreads();
        ++n_bar;
    };

    // ---- the segments ---------------------------------------------------------
    f32x16 sa[NBLK], sb[NBLK];
    for (int sg = 0; sg < nseg; ++sg) {
        const int q = sg == 0 ? seg_q0 : seg_q1;
        const int t0 = sg == 0 ? seg_a0 : seg_a1;
        const int t1 = sg == 0 ? seg_b0 : seg_b1;
        const bool out = sg == 0 ? seg_out0 : seg_out1;
        seg_end = t1;
        if (sg > 0) {  // the previous segment's last step may still read the buffers
            __syncthreads();
            ++n_bar;
        }
        begin_rows(q);
        if (t0 < t1) {
            // prologue: K tiles t0..t0+KD-1, V tiles t0..t0+VD-1 resident, Sᵀ(t0)
#pragma unroll
            for (int k = 0; k < KD; ++k)
#pragma unroll
                for (int i = 0; i < NLD; ++i) load_one(t0 + k, 0, k, 0, i);
#pragma unroll
            for (int k = 0; k < VD; ++k)
#pragma unroll
                for (int i = NLD; i < 2 * NLD; ++i) load_one(0, t0 + k, 0, k, i);
            load_mask(t0);
            __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): Q and the first tiles
            __syncthreads();
            ++n_bar;
            {
                const T* k0 = lds_k;
                op_t fr[PF + 1];
#pragma unroll
                for (int f = 0; f < PF; ++f) fr[f] = fetch_k(k0, f);
#pragma unroll
                for (int i = 0; i < N1; ++i) {
                    if (i + PF < N1) fr[(i + PF) % (PF + 1)] = fetch_k(k0, i + PF);
                    if constexpr (ACC_A) {
                        if (i < NBLK)
                            mfma_zero_qa(sa[i % NBLK], fr[i % (PF + 1)], qv[i / NBLK]);
                        else
                            mfma_acc_qa(sa[i % NBLK], fr[i % (PF + 1)], qv[i / NBLK]);
                    } else {
                        if (i < NBLK)
                            mfma_zero(sa[i % NBLK], fr[i % (PF + 1)], qv[i / NBLK]);
                        else
                            mfma_acc(sa[i % NBLK], fr[i % (PF + 1)], qv[i / NBLK]);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
            // the first softmax reads these accumulators right away: wait out
            // the MFMA result latency (the products are assembly, so the
            // compiler does not insert these wait states itself)
            asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7");
            // step t0 reloads the buffer K tile t0 was read from
            __syncthreads();
            ++n_bar;
            mask_tile(sa, t0);
            if constexpr (MK != 0) {
#pragma unroll
                for (int mj = 0; mj < NF / 8; ++mj) apply_mask(sa, read_mask(mj), mj, 0, 8);
            }
#pragma unroll
            for (int k = 0; k < NMX; ++k) max_item(sa, k);
            fin0();

            // steps t0 .. t1-2, two per iteration: S alternates between sa
            // and sb, and every buffer index is a constant
            int t = t0;
            for (; t + 2 < t1; t += 2) {
                step(t, 0, sa, sb, true);
                end_step();
                step(t + 1, 1, sb, sa, true);
                end_step();
            }
            if (t + 1 < t1) {
                step(t, 0, sa, sb, true);
                end_step();
                ++t;
                // S(t) to the registers the last step reads; after the
                // barrier, long after the MFMAs that wrote it
#pragma unroll
                for (int blk = 0; blk < NBLK; ++blk) {
                    asm volatile("" : "+v"(sb[blk]));
                    sa[blk] = sb[blk];
                }
            }
            // last step (t = t1-1): no next tile
            step(t, (t - t0) & 1, sa, sb, false);
            // the output accumulators were last written by MFMAs issued just
            // now (wait states as after the prologue); every accumulator
            // register stays allocated until then, also the padding dims'
            // ones that are never stored (D < DL), so that no other value
            // takes a register an MFMA is still writing
            asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7");
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
                if constexpr (ACC_A)
                    keep_acc_a(oacc[db]);
                else
                    keep_acc(oacc[db]);
            }
        }
        if (out) write_rows();
    }
    // every wavefront passes the same number of barriers
    for (; n_bar < bars_all; ++n_bar) __syncthreads();

    // ---- merge the heavy block's two partial states ------------------------
    // Group 1 leaves (m, l, O) of the heavy block's last nb tiles in LDS (the
    // tile buffers, idle now); group 0 combines them with its own:
    // m = max(m0, m1), O = O0·2^(m0-m) + O1·2^(m1-m), likewise the sums.
    if constexpr (NG == 2) {
        if (nb > 0) {
            // The last step of each segment ends without a barrier, and the
            // padding above adds none to the group with the most barriers:
            // wait until every wavefront has finished reading its tiles
            // before group 1 overwrites its own tile region (nb is uniform
            // over the workgroup, so all eight wavefronts arrive here).
            __syncthreads();
            constexpr int GRP_E = 2 * NBUF * TILE_E;  // elements per group region
            // both groups' tile regions are free now: group 1's O at the
            // start, then its (m, l, l_lse)
            constexpr int STASH_O = 4 * NDB * 16 * 64;  // floats
            float* stash_o = reinterpret_cast<float*>(lds);
            float* stash_s = stash_o + STASH_O;
            static_assert((STASH_O + 4 * 3 * 64) * 4 <= NG * GRP_E * ES, "merge stash fits the tile regions");
            if (grp == 1) {
#pragma unroll
                for (int db = 0; db < NDB; ++db)
#pragma unroll
                    for (int i = 0; i < 16; ++i) stash_o[((w4 * NDB + db) * 16 + i) * 64 + lane] = oacc[db][i];
                stash_s[(w4 * 3 + 0) * 64 + lane] = m_run;
                stash_s[(w4 * 3 + 1) * 64 + lane] = l_run;
                stash_s[(w4 * 3 + 2) * 64 + lane] = l_lse;
            }
            __syncthreads();
            if (grp == 0) {
                const float m1 = stash_s[(w4 * 3 + 0) * 64 + lane];
                const float l1 = stash_s[(w4 * 3 + 1) * 64 + lane];
                const float e1 = stash_s[(w4 * 3 + 2) * 64 + lane];
                const float m = fmaxf(m_run, m1);
                const float a0 = m == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m_run - m);
                const float a1 = m == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m1 - m);
#pragma unroll
                for (int db = 0; db < NDB; ++db)
#pragma unroll
                    for (int i = 0; i < 16; ++i)
                        oacc[db][i] = oacc[db][i] * a0 + stash_o[((w4 * NDB + db) * 16 + i) * 64 + lane] * a1;
                l_run = l_run * a0 + l1 * a1;
                l_lse = l_lse * a0 + e1 * a1;
                m_run = m;
                write_rows();
            }
        }
    }
}

template <typename T, int D, bool CAUSAL, bool PAD, bool LSE, bool ROPE, int MK = 0>
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
    kp.rope_pos = a.rope_pos;
    kp.rope_r1 = std::exp2(-2.0 * a.rope_lb / D);
    kp.cu = a.cu_seqlens;
    kp.total = int(a.total);
    kp.mask = a.mask;
    kp.mask_b = a.mask_b;
    kp.mask_h = a.mask_h;
    kp.inv_scale = 1.0f / a.scale;
    constexpr int NG = Groups<T, D, CAUSAL>::value;
    const int n_tasks = NG == 2 ? (kp.n_qb + 1) / 2 : kp.n_qb;
    const int64_t n_wg = int64_t(n_tasks) * kp.n_units;
    attn_detail::log_launch("attn_fwd_kernel<%s, D=%d, causal=%d, pad=%d, lse=%d, rope=%d, mask=%d> groups=%d "
                            "grid=%lld block=%d xcd_chunk=%d packed=%d B=%lld S=%lld Hq=%lld Hkv=%lld",
                            attn_detail::dtype_name(a.dtype), D, int(CAUSAL), int(PAD), int(LSE), int(ROPE), MK, NG,
                            (long long)n_wg, kThreads * NG, kp.xcd_chunk, a.cu_seqlens ? 1 : 0, (long long)a.B,
                            (long long)a.S, (long long)a.Hq, (long long)a.Hkv);
    hipLaunchKernelGGL((attn_fwd_kernel<T, D, CAUSAL, PAD, LSE, ROPE, MK>), dim3(unsigned(n_wg)), dim3(kThreads * NG), 0,
                       static_cast<hipStream_t>(a.stream), kp);
    const hipError_t e = hipGetLastError();
    if (e == hipSuccess) return ATTN_OK;
    if (e == hipErrorNoBinaryForGpu || e == hipErrorInvalidDeviceFunction) return ATTN_ERR_DEVICE;
    return ATTN_ERR_LAUNCH;
}

template <typename T, int D, bool LSE, bool ROPE>
int launch_r(const attn_detail::LaunchArgs& a) {
    if (a.causal) return a.padded ? launch_t<T, D, true, true, LSE, ROPE>(a) : launch_t<T, D, true, false, LSE, ROPE>(a);
    return a.padded ? launch_t<T, D, false, true, LSE, ROPE>(a) : launch_t<T, D, false, false, LSE, ROPE>(a);
}

template <typename T, int D, bool LSE>
int launch_l(const attn_detail::LaunchArgs& a) {
    return a.rope ? launch_r<T, D, LSE, true>(a) : launch_r<T, D, LSE, false>(a);
}

// with a mask tensor (16-bit types; no key padding, no rotary embedding)
template <typename T, int D, int MK>
int launch_mask_k(const attn_detail::LaunchArgs& a) {
    if (a.causal)
        return a.lse ? launch_t<T, D, true, false, true, false, MK>(a) : launch_t<T, D, true, false, false, false, MK>(a);
    return a.lse ? launch_t<T, D, false, false, true, false, MK>(a) : launch_t<T, D, false, false, false, false, MK>(a);
}

template <typename T, int D>
int launch_mask_d(const attn_detail::LaunchArgs& a) {
    return a.mask_bool ? launch_mask_k<T, D, 2>(a) : launch_mask_k<T, D, 1>(a);
}

// head dims without the rotary-embedding entry point (80, 96, 112)
template <typename T, int D>
int launch_d_plain(const attn_detail::LaunchArgs& a) {
    return a.lse != nullptr ? launch_r<T, D, true, false>(a) : launch_r<T, D, false, false>(a);
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
