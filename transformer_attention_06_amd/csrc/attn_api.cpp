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

namespace {

bool valid_dtype(int32_t dt) { return dt == ATTN_F32 || dt == ATTN_F16 || dt == ATTN_BF16; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

extern "C" int attn_fwd(const attn_tensor_t* q, const attn_tensor_t* k, const attn_tensor_t* v,
                        int mask_kind, const int32_t* pad_lens, float scale, int causal,
                        int n_q_heads, int n_kv_heads, const attn_tensor_t* out, float* lse,
                        void* stream) {
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

    if (q->D != 64 && q->D != 128) return ATTN_ERR_UNSUPPORTED;

    const int64_t B = q->B, S = q->S, D = q->D;
    if (B == 0 || S == 0) return ATTN_OK;  // empty input: nothing to launch

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

    attn_detail::LaunchArgs a;
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
    return attn_detail::launch(a);
}

extern "C" const char* attn_strerror(int code) {
    switch (code) {
        case ATTN_OK: return "success";
        case ATTN_ERR_NULL: return "a required pointer is NULL";
        case ATTN_ERR_SHAPE: return "B, S or D disagree between q, k, v, out (or are negative)";
        case ATTN_ERR_HEADS: return "head counts disagree with the tensors, or n_q_heads % n_kv_heads != 0";
        case ATTN_ERR_DTYPE: return "unknown dtype, or q, k, v, out are not all the same dtype";
        case ATTN_ERR_UNSUPPORTED: return "unsupported size: D must be 64 or 128, and sizes within the documented limits";
        case ATTN_ERR_MASK: return "bad mask arguments: mask_kind unknown, pad_lens NULL/non-NULL mismatch, or causal not 0/1";
        case ATTN_ERR_ALIGN: return "a data pointer is not 16-byte aligned (pad_lens/lse: 4-byte)";
        case ATTN_ERR_LAUNCH: return "the HIP kernel launch failed";
        case ATTN_ERR_DEVICE: return "the current device cannot run this library's gfx950 code";
        default: return "unknown error code";
    }
}

extern "C" const char* attn_version(void) { return "attn_fwd 0.1.0 gfx950"; }
