// attn_launch.h — internal interface between the validated C ABI and the
// kernel launcher (not part of the public ABI).
#pragma once

#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstdlib>

#include "attn_fwd.h"

namespace attn_detail {

// ATTN_LOG set to a value other than "" or "0": every launch prints one line
// on stderr naming its kernel variant (template arguments), grid and
// workgroup size, before the launch.
inline bool log_on() {
    static const bool on = [] {
        const char* e = std::getenv("ATTN_LOG");
        return e && e[0] && !(e[0] == '0' && e[1] == 0);
    }();
    return on;
}

inline void log_launch(const char* fmt, ...) {
    if (!log_on()) return;
    va_list ap;
    va_start(ap, fmt);
    std::fputs("[attn] ", stderr);
    std::vfprintf(stderr, fmt, ap);
    std::fputc('\n', stderr);
    va_end(ap);
}

// name of an attn_dtype_t value
inline const char* dtype_name(int32_t dt) { return dt == 2 ? "bf16" : dt == 1 ? "fp16" : "fp32"; }

// Query rows owned by one workgroup (4 wavefronts x 32 rows).
constexpr int kBlockM = 128;

struct LaunchArgs {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    float* lse;
    const int32_t* pad_lens;
    int32_t dtype;
    int64_t B, S, Hq, Hkv, D;
    int causal;
    int padded;
    float scale;
    void* stream;
    // rotary embedding of Q inside the attention kernel (K is rotated
    // beforehand by launch_rope_k)
    int rope = 0;
    const int32_t* rope_pos = nullptr;  // (B, S) positions or null (0..S-1)
    double rope_f[64] = {};             // theta_i / 2pi for i < D/2
    double rope_lb = 0.0;               // log2(base): theta_i = 2^(-2i/D * rope_lb)
    // packed sequences: B sequences at rows [cu[b], cu[b+1]) of (1, total,
    // H, D) buffers; S is then the longest length and lse is (Hq, total)
    const int32_t* cu_seqlens = nullptr;
    int64_t total = 0;
    // additive mask (Bm, Hm, S, S) in the input type; mask_b / mask_h are 1
    // when the mask has a batch dimension of B / a head dimension of Hq
    const void* mask = nullptr;
    int mask_b = 0, mask_h = 0;
    int mask_bool = 0;  // 1: one byte per entry, nonzero = the key takes part
};

// Enqueue the kernel; returns ATTN_OK or ATTN_ERR_LAUNCH / ATTN_ERR_DEVICE.
int launch(const LaunchArgs& a);
// the same per element type and head dim (one translation unit each)
int launch_fwd_bf16_d64(const LaunchArgs& a);
int launch_fwd_bf16_d128(const LaunchArgs& a);
int launch_fwd_f16_d64(const LaunchArgs& a);
int launch_fwd_f16_d128(const LaunchArgs& a);
int launch_fwd_f32_d64(const LaunchArgs& a);
int launch_fwd_f32_d128(const LaunchArgs& a);
// head dims 80, 96, 112, 144, 160, 192, 256 (16-bit types; no rotary embedding)
int launch_fwd_bf16_d192(const LaunchArgs& a);
int launch_fwd_bf16_d256(const LaunchArgs& a);
int launch_fwd_f16_d192(const LaunchArgs& a);
int launch_fwd_f16_d256(const LaunchArgs& a);
int launch_fwd_bf16_d144(const LaunchArgs& a);
int launch_fwd_bf16_d160(const LaunchArgs& a);
int launch_fwd_f16_d144(const LaunchArgs& a);
int launch_fwd_f16_d160(const LaunchArgs& a);
int launch_fwd_bf16_d80(const LaunchArgs& a);
int launch_fwd_bf16_d96(const LaunchArgs& a);
int launch_fwd_bf16_d112(const LaunchArgs& a);
int launch_fwd_f16_d80(const LaunchArgs& a);
int launch_fwd_f16_d96(const LaunchArgs& a);
int launch_fwd_f16_d112(const LaunchArgs& a);
// head dims the tuned kernel serves for this element type
inline bool tuned_head_dim(int32_t dtype, int64_t D) {
    return D == 64 || D == 128 ||
           (dtype != ATTN_F32 && (D == 80 || D == 96 || D == 112 || D == 144 || D == 160 || D == 192 || D == 256));
}

// The tuned kernel with a mask tensor (a.mask; 16-bit types, D = 64 or 128,
// rows of 16-byte multiples, planes under 2^31 bytes).
int launch_masked_tuned(const LaunchArgs& a);
int launch_fwd_mask_bf16_d64(const LaunchArgs& a);
int launch_fwd_mask_bf16_d128(const LaunchArgs& a);
int launch_fwd_mask_f16_d64(const LaunchArgs& a);
int launch_fwd_mask_f16_d128(const LaunchArgs& a);

// Enqueue the attention with an additive mask tensor (16-bit types only).
int launch_masked(const LaunchArgs& a);

// Enqueue the general kernel (16-bit types; head dims that are multiples of
// 16 up to 256) without a mask tensor.
int launch_general(const LaunchArgs& a);

// Enqueue the rotary embedding of K (a.k, layout (B, S, Hkv, D)) into
// k_out (same layout; may be a.k itself) with a.rope_pos and a.rope_f.
int launch_rope_k(const LaunchArgs& a, void* k_out);

// Decode attention over a KV cache (split over key chunks, then merged).
struct DecodeArgs {
    const void* q;             // (B, Sq, Hq, D)
    const void* k;             // (B, Sk, Hkv, D)
    const void* v;
    void* o;                   // (B, Sq, Hq, D)
    float* lse;                // (B, Hq, Sq) or null
    const int32_t* cache_lens; // int32[B] or null (= Sk)
    void* workspace;           // decode_workspace_bytes(...) bytes, 16-byte aligned
    int32_t dtype;
    int64_t B, Sq, Sk, Hq, Hkv, D;
    int causal;
    int n_split;
    float scale;
    void* stream;
};

// Key chunks a cache of Sk rows is split into (at least one; defined for
// every Sk >= 0 without overflow).
int64_t decode_splits(int64_t Sk);

// Size of the fixed device workspace of the allocation-free decode entry
// point (one array per GPU, shared by every call on that GPU).
constexpr int64_t kDecodeScratchBytes = int64_t(32) << 20;

// Every decode workspace starts with this many bytes of arrival counters
// (one int per (batch, kv head, group of query rows) of a split launch; a
// launch with more than one split has fewer than 256 such groups), zero
// before a call and zero again after it; the partial results follow.
constexpr int64_t kDecodeCounterBytes = 1024;

// This device's address of that workspace (looked up on the first call on
// each device); ATTN_OK or ATTN_ERR_DEVICE.
int decode_scratch(void** ws);

// Enqueue the split and merge kernels.
int launch_decode(const DecodeArgs& a);

}  // namespace attn_detail
