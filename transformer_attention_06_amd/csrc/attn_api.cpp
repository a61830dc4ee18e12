// attn_api.cpp — argument validation and dispatch for attn_fwd (C ABI).
//
// The host side of the fused operator follows the wrapper duties that
// "ops-transformer：Transformer算子融合与推理加速实战" §3.2 lists: parse and
// check the parameters, choose the tiling from the shapes, pack pointers and
// sizes into one launch-parameter struct, and launch.  Every check here runs
// before any HIP call, so a rejected call leaves the device untouched (shape
// errors surface as clear error codes, §6.2).
#include "attn_fwd.h"
#include "attn_launch.h"

#include <cmath>
#include <cstdint>
#include <initializer_list>

namespace {

bool valid_dtype(int32_t dt) { return dt == ATTN_F32 || dt == ATTN_F16 || dt == ATTN_BF16; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Checks every argument of attn_fwd and fills the launch struct; `empty` is
// set when there is nothing to launch (B == 0 or S == 0).
// general_d: head dims other than 64 and 128 (multiples of 16 up to 256,
// 16-bit types) are accepted; they run on the general kernel.
int prepare(const attn_tensor_t* q, const attn_tensor_t* k, const attn_tensor_t* v, int mask_kind,
            const int32_t* pad_lens, float scale, int causal, int n_q_heads, int n_kv_heads,
            const attn_tensor_t* out, float* lse, void* stream, attn_detail::LaunchArgs& a, bool& empty,
            bool general_d = false) {
    empty = false;
    if (!q || !k || !v || !out) return ATTN_ERR_NULL;
    if (!valid_dtype(q->dtype) || !valid_dtype(k->dtype) || !valid_dtype(v->dtype) ||
        !valid_dtype(out->dtype))
        return ATTN_ERR_DTYPE;
    if (k->dtype != q->dtype || v->dtype != q->dtype || out->dtype != q->dtype) return ATTN_ERR_DTYPE;

    const attn_tensor_t* all[4] = {q, k, v, out};
    for (const attn_tensor_t* t : all)
        if (t->B < 0 || t->S < 0 || t->H < 0 || t->D < 0) return ATTN_ERR_SHAPE;
    for (const attn_tensor_t* t : all)
        if (t->B != q->B || t->S != q->S || t->D != q->D) return ATTN_ERR_SHAPE;

    if (n_q_heads <= 0 || n_kv_heads <= 0) return ATTN_ERR_HEADS;
    if (q->H != n_q_heads || out->H != n_q_heads) return ATTN_ERR_HEADS;
    if (k->H != n_kv_heads || v->H != n_kv_heads) return ATTN_ERR_HEADS;
    if (n_q_heads % n_kv_heads != 0) return ATTN_ERR_HEADS;
    if (n_q_heads > 65535) return ATTN_ERR_UNSUPPORTED;

    if (causal != 0 && causal != 1) return ATTN_ERR_MASK;
    if (mask_kind == ATTN_MASK_NONE) {
        if (pad_lens != nullptr) return ATTN_ERR_MASK;
    } else if (mask_kind == ATTN_MASK_KEY_PADDING) {
        if (pad_lens == nullptr) return ATTN_ERR_MASK;
        if ((reinterpret_cast<uintptr_t>(pad_lens) & 3u) != 0) return ATTN_ERR_ALIGN;
    } else {
        return ATTN_ERR_MASK;
    }

    const bool d_tuned = q->D == 64 || q->D == 128;
    const bool d_general = general_d && q->dtype != ATTN_F32 && q->D % 16 == 0 && q->D >= 16 && q->D <= 256;
    if (!d_tuned && !d_general) return ATTN_ERR_UNSUPPORTED;

    const int64_t B = q->B, S = q->S, D = q->D;
    if (B == 0 || S == 0) {  // empty input: nothing to launch
        empty = true;
        return ATTN_OK;
    }

    if (S >= (int64_t(1) << 29)) return ATTN_ERR_UNSUPPORTED;
    // Total element counts must stay far from int64 overflow.
    const double elems = double(B) * double(S) * double(n_q_heads) * double(D);
    if (elems >= 4.0e18) return ATTN_ERR_UNSUPPORTED;
    // K/V of one batch are addressed with 32-bit byte offsets on the device.
    const int64_t esize = q->dtype == ATTN_F32 ? 4 : 2;
    if (S * int64_t(n_kv_heads) * D * esize >= (int64_t(1) << 31)) return ATTN_ERR_UNSUPPORTED;
    const int64_t n_qb = (S + attn_detail::kBlockM - 1) / attn_detail::kBlockM;
    const double wgs = double(n_qb) * double(n_q_heads) * double(B);
    if (wgs >= 2147483647.0) return ATTN_ERR_UNSUPPORTED;

    if (!q->data || !k->data || !v->data || !out->data) return ATTN_ERR_NULL;
    if (!aligned16(q->data) || !aligned16(k->data) || !aligned16(v->data) || !aligned16(out->data))
        return ATTN_ERR_ALIGN;
    if (lse && (reinterpret_cast<uintptr_t>(lse) & 3u) != 0) return ATTN_ERR_ALIGN;

    float sc = scale;
    if (!(sc > 0.0f) || !std::isfinite(sc)) sc = 1.0f / std::sqrt(float(D));

    a.q = q->data;
    a.k = k->data;
    a.v = v->data;
    a.o = out->data;
    a.lse = lse;
    a.pad_lens = pad_lens;
    a.dtype = q->dtype;
    a.B = B;
    a.S = S;
    a.Hq = n_q_heads;
    a.Hkv = n_kv_heads;
    a.D = D;
    a.causal = causal;
    a.padded = (mask_kind == ATTN_MASK_KEY_PADDING) ? 1 : 0;
    a.scale = sc;
    a.stream = stream;
    return ATTN_OK;
}

bool overlap(const void* p, int64_t pn, const void* r, int64_t rn) {
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(p), b0 = reinterpret_cast<uintptr_t>(r);
    return a0 < b0 + uintptr_t(rn) && b0 < a0 + uintptr_t(pn);
}

int64_t bytes_of(const attn_tensor_t* t) {
    return t->B * t->S * t->H * t->D * (t->dtype == ATTN_F32 ? 4 : 2);
}

}  // namespace

extern "C" int attn_fwd(const attn_tensor_t* q, const attn_tensor_t* k, const attn_tensor_t* v,
                        int mask_kind, const int32_t* pad_lens, float scale, int causal,
                        int n_q_heads, int n_kv_heads, const attn_tensor_t* out, float* lse,
                        void* stream) {
    attn_detail::LaunchArgs a;
    bool empty = false;
    const int rc = prepare(q, k, v, mask_kind, pad_lens, scale, causal, n_q_heads, n_kv_heads, out, lse,
                           stream, a, empty, true);
    if (rc != ATTN_OK || empty) return rc;
    if (attn_detail::tuned_head_dim(a.dtype, a.D)) return attn_detail::launch(a);
    // other head dims: the general kernel (one workgroup per batch, head and
    // 128-row block; batch on the grid's z axis)
    if (a.B > 65535) return ATTN_ERR_UNSUPPORTED;
    return attn_detail::launch_general(a);
}

// Packed variable-length sequences ([ATB-guide] §6.1 and §8.7: one
// attention operator over whatever lengths arrive; [ops-transformer] §5.2:
// batch and heads merged into one parallel axis, then the sequence split):
// the same kernel, each workgroup reading its sequence's offset and length.
extern "C" int attn_fwd_varlen(const attn_tensor_t* q, const attn_tensor_t* k, const attn_tensor_t* v,
                               const int32_t* cu_seqlens, int n_seqs, int64_t max_seqlen, float scale,
                               int causal, int n_q_heads, int n_kv_heads, const attn_tensor_t* out,
                               float* lse, void* stream) {
    attn_detail::LaunchArgs a;
    bool empty = false;
    const int rc = prepare(q, k, v, ATTN_MASK_NONE, nullptr, scale, causal, n_q_heads, n_kv_heads, out, lse,
                           stream, a, empty);
    if (rc != ATTN_OK) return rc;
    if (q->B != 1) return ATTN_ERR_SHAPE;  // packed: one (1, T, H, D) buffer per tensor
    if (n_seqs < 0 || max_seqlen < 0 || max_seqlen > q->S) return ATTN_ERR_SHAPE;
    if (!cu_seqlens) return ATTN_ERR_NULL;
    if ((reinterpret_cast<uintptr_t>(cu_seqlens) & 3u) != 0) return ATTN_ERR_ALIGN;
    if (empty || n_seqs == 0 || max_seqlen == 0) return ATTN_OK;
    const int64_t n_qb = (max_seqlen + attn_detail::kBlockM - 1) / attn_detail::kBlockM;
    if (double(n_seqs) * double(n_q_heads) >= 2147483647.0 ||
        double(n_qb) * double(n_q_heads) * double(n_seqs) >= 2147483647.0)
        return ATTN_ERR_UNSUPPORTED;
    a.total = a.S;
    a.B = n_seqs;
    a.S = max_seqlen;
    a.cu_seqlens = cu_seqlens;
    return attn_detail::launch(a);
}

// Explicit additive mask tensor ([graph-opt] Pattern 2's FlashAttention(Q, K,
// V, mask, scale); [ATB-guide] §8.2 passes the mask as one more FP16 input):
// a kernel of its own that reads the mask block of every tile.
extern "C" int attn_fwd_masked(const attn_tensor_t* q, const attn_tensor_t* k, const attn_tensor_t* v,
                               const void* mask, int mask_type, int64_t mask_B, int64_t mask_H, float scale,
                               int causal,
                               int n_q_heads, int n_kv_heads, const attn_tensor_t* out, float* lse,
                               void* stream) {
    attn_detail::LaunchArgs a;
    bool empty = false;
    const int rc = prepare(q, k, v, ATTN_MASK_NONE, nullptr, scale, causal, n_q_heads, n_kv_heads, out, lse,
                           stream, a, empty, true);
    if (rc != ATTN_OK) return rc;
    if (q->dtype == ATTN_F32) return ATTN_ERR_UNSUPPORTED;  // 16-bit types only
    if (mask_type != ATTN_MASK_ADDITIVE && mask_type != ATTN_MASK_BOOL) return ATTN_ERR_MASK;
    if (mask_B != 1 && mask_B != q->B) return ATTN_ERR_MASK;
    if (mask_H != 1 && mask_H != n_q_heads) return ATTN_ERR_MASK;
    if (empty) return ATTN_OK;
    if (!mask) return ATTN_ERR_NULL;
    if ((reinterpret_cast<uintptr_t>(mask) & 15u) != 0) return ATTN_ERR_ALIGN;
    if (q->B > 65535) return ATTN_ERR_UNSUPPORTED;  // grid z
    a.mask = mask;
    a.mask_b = mask_B != 1 ? 1 : 0;
    a.mask_h = mask_H != 1 ? 1 : 0;
    a.mask_bool = mask_type == ATTN_MASK_BOOL ? 1 : 0;
    // the tuned kernel stages 16-byte chunks of mask rows (8 additive entries
    // or 16 bytes) and addresses a mask plane with 32-bit offsets; other
    // shapes and head dims take the general kernel
    const int64_t me = a.mask_bool ? 1 : 2;
    if ((a.D == 64 || a.D == 128) && (a.S * me) % 16 == 0 && a.S * a.S * me < (int64_t(1) << 31))
        return attn_detail::launch_masked_tuned(a);
    return attn_detail::launch_masked(a);
}

// Rotary embedding of Q and K fused with the attention ([ATB-guide] §4.1,
// fifth fusion pattern; §8.4 for the rotation and its base of 10000): K is
// rotated once into k_rot by a bandwidth-bound pass, Q in registers inside
// the attention kernel as its tile is loaded.
extern "C" int attn_fwd_rope(const attn_tensor_t* q, const attn_tensor_t* k, const attn_tensor_t* v,
                             int mask_kind, const int32_t* pad_lens, float scale, int causal,
                             int n_q_heads, int n_kv_heads, const int32_t* positions, float rope_base,
                             const attn_tensor_t* k_rot, const attn_tensor_t* out, float* lse,
                             void* stream) {
    attn_detail::LaunchArgs a;
    bool empty = false;
    const int rc = prepare(q, k, v, mask_kind, pad_lens, scale, causal, n_q_heads, n_kv_heads, out, lse,
                           stream, a, empty);
    if (rc != ATTN_OK) return rc;
    if (!k_rot) return ATTN_ERR_NULL;
    if (!valid_dtype(k_rot->dtype) || k_rot->dtype != k->dtype) return ATTN_ERR_DTYPE;
    if (k_rot->B != k->B || k_rot->S != k->S || k_rot->H != k->H || k_rot->D != k->D) return ATTN_ERR_SHAPE;
    if (empty) return ATTN_OK;
    if (!k_rot->data) return ATTN_ERR_NULL;
    if (!aligned16(k_rot->data)) return ATTN_ERR_ALIGN;
    if (positions && (reinterpret_cast<uintptr_t>(positions) & 3u) != 0) return ATTN_ERR_ALIGN;
    // k_rot is written before the attention reads q, v and writes out: it may
    // be k itself, but must not overlap any other tensor (or k partially)
    const int64_t kb = bytes_of(k_rot);
    if (k_rot->data != k->data && overlap(k_rot->data, kb, k->data, bytes_of(k))) return ATTN_ERR_ALIAS;
    if (overlap(k_rot->data, kb, q->data, bytes_of(q)) || overlap(k_rot->data, kb, v->data, bytes_of(v)) ||
        overlap(k_rot->data, kb, out->data, bytes_of(out)))
        return ATTN_ERR_ALIAS;
    if (lse && overlap(k_rot->data, kb, lse, int64_t(sizeof(float)) * q->B * n_q_heads * q->S))
        return ATTN_ERR_ALIAS;
    double base = rope_base;
    if (!(base > 0.0) || !std::isfinite(base)) base = 10000.0;
    const int64_t D = q->D;
    for (int64_t i = 0; i < D / 2; ++i)
        a.rope_f[i] = std::pow(base, -2.0 * double(i) / double(D)) / (2.0 * 3.14159265358979323846);
    a.rope_lb = std::log2(base);
    a.rope_pos = positions;
    a.rope = 1;
    const int rk = attn_detail::launch_rope_k(a, k_rot->data);
    if (rk != ATTN_OK) return rk;
    a.k = k_rot->data;
    return attn_detail::launch(a);
}

// Decode attention over a KV cache: Sq new rows per sequence against the
// first cache_lens[b] cached rows, end-aligned causal rule (the ATB
// introduction's FlashAttention with KV-cache management; "CANN-ops-
// transformer和ATB…" passes the cache into FlashAttention every step).
extern "C" int64_t attn_decode_workspace_bytes(int64_t B, int64_t Sq, int n_q_heads, int64_t D, int64_t Sk) {
    if (B < 0 || Sq < 0 || n_q_heads < 0 || D < 0 || Sk < 0) return -1;
    // the counters, then n_split · B · Hq · Sq · 4 · (D + 3), or -1 where it
    // does not fit int64
    int64_t r = attn_detail::decode_splits(Sk);
    for (int64_t x : {B, int64_t(n_q_heads), Sq, int64_t(sizeof(float))})
        if (__builtin_mul_overflow(r, x, &r)) return -1;
    int64_t d3 = 0;
    if (__builtin_add_overflow(D, int64_t(3), &d3) || __builtin_mul_overflow(r, d3, &r)) return -1;
    if (__builtin_add_overflow(r, attn_detail::kDecodeCounterBytes, &r)) return -1;
    return r;
}

// Argument checks and launch parameters shared by the two decode entry
// points (no HIP call).  *need receives the workspace bytes; a returned
// ATTN_OK with a->B == 0 or a->Sq == 0 means there is nothing to launch.
static int decode_prepare(const attn_tensor_t* q, const attn_tensor_t* k_cache, const attn_tensor_t* v_cache,
                          const int32_t* cache_lens, float scale, int causal, int n_q_heads, int n_kv_heads,
                          const attn_tensor_t* out, float* lse, void* stream, attn_detail::DecodeArgs* a,
                          int64_t* need) {
    if (!q || !k_cache || !v_cache || !out) return ATTN_ERR_NULL;
    const attn_tensor_t* all[4] = {q, k_cache, v_cache, out};
    for (const attn_tensor_t* t : all)
        if (!valid_dtype(t->dtype)) return ATTN_ERR_DTYPE;
    for (const attn_tensor_t* t : all)
        if (t->dtype != q->dtype) return ATTN_ERR_DTYPE;
    for (const attn_tensor_t* t : all)
        if (t->B < 0 || t->S < 0 || t->H < 0 || t->D < 0) return ATTN_ERR_SHAPE;
    if (k_cache->B != q->B || v_cache->B != q->B || out->B != q->B) return ATTN_ERR_SHAPE;
    if (k_cache->D != q->D || v_cache->D != q->D || out->D != q->D) return ATTN_ERR_SHAPE;
    if (v_cache->S != k_cache->S || out->S != q->S) return ATTN_ERR_SHAPE;
    if (n_q_heads <= 0 || n_kv_heads <= 0) return ATTN_ERR_HEADS;
    if (q->H != n_q_heads || out->H != n_q_heads) return ATTN_ERR_HEADS;
    if (k_cache->H != n_kv_heads || v_cache->H != n_kv_heads) return ATTN_ERR_HEADS;
    if (n_q_heads % n_kv_heads != 0 || n_q_heads > 65535) return n_q_heads > 65535 ? ATTN_ERR_UNSUPPORTED
                                                                                    : ATTN_ERR_HEADS;
    if (causal != 0 && causal != 1) return ATTN_ERR_MASK;
    if (cache_lens && (reinterpret_cast<uintptr_t>(cache_lens) & 3u) != 0) return ATTN_ERR_ALIGN;
    if (q->D != 64 && q->D != 128) return ATTN_ERR_UNSUPPORTED;
    const int64_t B = q->B, Sq = q->S, Sk = k_cache->S, D = q->D;
    a->B = B;
    a->Sq = Sq;
    *need = 0;
    if (B == 0 || Sq == 0) return ATTN_OK;  // no query row: nothing to launch
    if (Sk >= (int64_t(1) << 29) || Sq >= (int64_t(1) << 20)) return ATTN_ERR_UNSUPPORTED;
    if (B > 65535 || B * n_kv_heads > 65535) return ATTN_ERR_UNSUPPORTED;
    const int64_t rows_per_kv = int64_t(n_q_heads / n_kv_heads) * Sq;
    if ((rows_per_kv + 7) / 8 > 65535) return ATTN_ERR_UNSUPPORTED;
    if (B * n_q_heads * Sq / 4 + 1 >= int64_t(1) << 31) return ATTN_ERR_UNSUPPORTED;
    *need = attn_decode_workspace_bytes(B, Sq, n_q_heads, D, Sk);
    if (*need < 0) return ATTN_ERR_UNSUPPORTED;  // the workspace size does not fit int64
    if (!q->data || !out->data) return ATTN_ERR_NULL;
    if (Sk > 0 && (!k_cache->data || !v_cache->data)) return ATTN_ERR_NULL;
    if (!aligned16(q->data) || !aligned16(out->data) ||
        (Sk > 0 && (!aligned16(k_cache->data) || !aligned16(v_cache->data))))
        return ATTN_ERR_ALIGN;
    if (lse && (reinterpret_cast<uintptr_t>(lse) & 3u) != 0) return ATTN_ERR_ALIGN;
    float sc = scale;
    if (!(sc > 0.0f) || !std::isfinite(sc)) sc = 1.0f / std::sqrt(float(D));
    a->q = q->data;
    a->k = k_cache->data;
    a->v = v_cache->data;
    a->o = out->data;
    a->lse = lse;
    a->cache_lens = cache_lens;
    a->workspace = nullptr;
    a->dtype = q->dtype;
    a->Sk = Sk;
    a->Hq = n_q_heads;
    a->Hkv = n_kv_heads;
    a->D = D;
    a->causal = causal;
    a->n_split = int(attn_detail::decode_splits(Sk));  // Sk < 2^29: fits
    a->scale = sc;
    a->stream = stream;
    return ATTN_OK;
}

extern "C" int attn_fwd_decode(const attn_tensor_t* q, const attn_tensor_t* k_cache,
                               const attn_tensor_t* v_cache, const int32_t* cache_lens, float scale,
                               int causal, int n_q_heads, int n_kv_heads, const attn_tensor_t* out,
                               float* lse, void* workspace, int64_t workspace_bytes, void* stream) {
    attn_detail::DecodeArgs a;
    int64_t need = 0;
    const int rc = decode_prepare(q, k_cache, v_cache, cache_lens, scale, causal, n_q_heads, n_kv_heads, out, lse,
                                  stream, &a, &need);
    if (rc != ATTN_OK || a.B == 0 || a.Sq == 0) return rc;
    if (!workspace) return ATTN_ERR_NULL;
    if (workspace_bytes < need) return ATTN_ERR_WORKSPACE;
    if (!aligned16(workspace)) return ATTN_ERR_ALIGN;
    a.workspace = workspace;
    return attn_detail::launch_decode(a);
}

// The same decode without any allocation: the workspace is the library's
// fixed per-GPU array (attn_detail::decode_scratch).  Checks first, then the
// size limit, then the one-time address lookup, then the two launches.
extern "C" int attn_fwd_decode_noalloc(const attn_tensor_t* q, const attn_tensor_t* k_cache,
                                       const attn_tensor_t* v_cache, const int32_t* cache_lens, float scale,
                                       int causal, int n_q_heads, int n_kv_heads, const attn_tensor_t* out,
                                       float* lse, void* stream) {
    attn_detail::DecodeArgs a;
    int64_t need = 0;
    int rc = decode_prepare(q, k_cache, v_cache, cache_lens, scale, causal, n_q_heads, n_kv_heads, out, lse, stream,
                            &a, &need);
    if (rc != ATTN_OK || a.B == 0 || a.Sq == 0) return rc;
    if (need > attn_detail::kDecodeScratchBytes) return ATTN_ERR_SCRATCH;
    rc = attn_detail::decode_scratch(&a.workspace);
    if (rc != ATTN_OK) return rc;
    return attn_detail::launch_decode(a);
}

extern "C" const char* attn_strerror(int code) {
    switch (code) {
        case ATTN_OK: return "success";
        case ATTN_ERR_NULL: return "a required pointer is NULL";
        case ATTN_ERR_SHAPE: return "B, S or D disagree between q, k, v, out (or are negative)";
        case ATTN_ERR_HEADS: return "head counts disagree with the tensors, or n_q_heads % n_kv_heads != 0";
        case ATTN_ERR_DTYPE: return "unknown dtype, or q, k, v, out are not all the same dtype";
        case ATTN_ERR_UNSUPPORTED: return "unsupported size or type: D must be 64 or 128 (attn_fwd and attn_fwd_masked: a multiple of 16 in [16, 256] for fp16/bf16), and sizes within the documented limits";
        case ATTN_ERR_MASK: return "bad mask arguments: mask_kind unknown, pad_lens NULL/non-NULL mismatch, or causal not 0/1";
        case ATTN_ERR_ALIGN: return "a data pointer is not 16-byte aligned (pad_lens/lse: 4-byte)";
        case ATTN_ERR_LAUNCH: return "the HIP kernel launch failed";
        case ATTN_ERR_DEVICE: return "the current device cannot run this library's gfx950 code";
        case ATTN_ERR_ALIAS: return "k_rot overlaps q, v, out, lse, or part of k (it may be k itself)";
        case ATTN_ERR_WORKSPACE: return "workspace smaller than attn_decode_workspace_bytes() requires";
        case ATTN_ERR_SCRATCH: return "attn_fwd_decode_noalloc: these sizes need more workspace than its fixed 32 MiB per GPU (attn_decode_workspace_bytes() > 33554432); use attn_fwd_decode with a caller workspace";
        default: return "unknown error code";
    }
}

#ifndef ATTN_SRC_HASH
#define ATTN_SRC_HASH "unknown"
#endif

// The version string ends with the hash of the sources the library was built
// from (set by the build), so a caller can tell which sources it runs.
extern "C" const char* attn_version(void) { return "attn_fwd 0.2.0 gfx950 src " ATTN_SRC_HASH; }
