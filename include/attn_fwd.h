/*
 * attn_fwd.h — C ABI of the MI355X (gfx950) fused attention forward library
 * (libattn_fwd.so).
 *
 * The operation (one call = one fused kernel launch):
 *
 *   for every batch b and query head h, with kv head g = floor(h*Hkv/Hq):
 *     S    = (Q[b,:,h,:] · K[b,:,g,:]ᵀ) · scale
 *     S_ij = -inf where key j is masked (causal: j > i; key padding: j >= L_b)
 *     P    = softmax(S) along keys;   O[b,:,h,:] = P · V[b,:,g,:]
 *     LSE  = ln(sum_j exp(S_ij))      (natural log of the scaled scores)
 *
 * This is the chain "Q·Kᵀ → Scale → Mask → Softmax → Drop → ·V" that the page
 * "CANN-ATB图优化-昇腾NPU怎么把PyTorch计算图改造成融合算子" (Pattern 2, SDPA →
 * FlashAttention) replaces by one FlashAttention(Q, K, V, mask, scale) call,
 * with dropout as the identity (inference forward).  The kernel computes it
 * blockwise with an online softmax, as "ops-transformer：Transformer算子融合与
 * 推理加速实战" §2.2 and §3.2 describe: the S×S score matrix never reaches
 * device memory.  The call parameters (scale, mask type, whether to output the
 * intermediate LSE) follow the same page's §4.2; the head counts and the
 * causal flag follow the MhaV3 parameters of the ATB engineering guide
 * (hwcomputing.csdn.net/6a59a88310ee7a33f28e5ce9) §8.2.
 *
 * Conventions
 *   - Layout: every tensor is contiguous (B, S, H, D), row-major, D fastest
 *     ("ops-transformer…" §2.3/§4.2).  q and out have H = n_q_heads; k and v
 *     have H = n_kv_heads.  q, k, v share B, S and D (self-attention).
 *   - Pointers are DEVICE pointers (HIP), except the descriptor structs
 *     themselves, which are host memory read during the call only.
 *   - Ownership: the caller allocates and owns every buffer.  The library
 *     never allocates, frees or synchronises device memory and keeps no
 *     state between calls; it is re-entrant and thread-safe.
 *   - Asynchrony: the kernel is enqueued on `stream` (a hipStream_t; NULL =
 *     the default stream).  ATTN_OK means "enqueued"; a device-side fault
 *     surfaces at the caller's next synchronisation.
 *   - Validation: every argument check runs on the host before any HIP call,
 *     so an error return leaves the device untouched.  B == 0 or S == 0
 *     returns ATTN_OK without a launch ("ops-transformer…" §6.4: empty input).
 *   - Supported: dtype fp32, fp16, bf16 (q, k, v and out all the same);
 *     D in {64, 128} on every entry point.  The page "CANN-ops-transformer和
 *     ATB-昇腾NPU上算子和加速库怎么配合" gates its fused kernel on a head_dim
 *     that is a multiple of 16: attn_fwd and attn_fwd_masked also take fp16 /
 *     bf16 with D a multiple of 16 in [16, 256] (a second, general kernel:
 *     the head dim padded to a multiple of 32 in registers and LDS, not in
 *     memory; B <= 65535).  Other D return ATTN_ERR_UNSUPPORTED: there is no
 *     fallback path.
 *   - Precision: 16-bit inputs run both products on bf16/fp16 MFMA with fp32
 *     accumulation; the running max, running sum and output accumulator are
 *     fp32 and the output is rounded to the input dtype only at the end
 *     ("ops-transformer…" §2.4).  The probabilities P are rounded to the input
 *     dtype before the P·V product.  fp32 inputs keep everything in fp32.
 */
#ifndef ATTN_FWD_H
#define ATTN_FWD_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    ATTN_F32 = 0,
    ATTN_F16 = 1,
    ATTN_BF16 = 2
} attn_dtype_t;

typedef enum {
    ATTN_MASK_NONE = 0,        /* no padding mask                              */
    ATTN_MASK_KEY_PADDING = 1  /* batch b sees keys j < pad_lens[b] only       */
} attn_mask_kind_t;

/* Element type of attn_fwd_masked's mask tensor. */
typedef enum {
    ATTN_MASK_ADDITIVE = 0,  /* q's dtype, added to the scaled scores (-inf hides) */
    ATTN_MASK_BOOL = 1       /* one byte per entry: nonzero = the key takes part */
} attn_mask_type_t;

/* Tensor descriptor: a contiguous (B, S, H, D) device buffer. */
typedef struct {
    void*   data;   /* device pointer, 16-byte aligned                        */
    int32_t dtype;  /* attn_dtype_t                                            */
    int64_t B, S, H, D;
} attn_tensor_t;

/* Return codes (0 = success, negative = error). */
enum {
    ATTN_OK = 0,
    ATTN_ERR_NULL = -1,        /* a required pointer is NULL                   */
    ATTN_ERR_SHAPE = -2,       /* B/S/D disagree between tensors, or negative  */
    ATTN_ERR_HEADS = -3,       /* head counts disagree or Hq % Hkv != 0        */
    ATTN_ERR_DTYPE = -4,       /* unknown dtype or tensors of mixed dtype      */
    ATTN_ERR_UNSUPPORTED = -5, /* D not in {64, 128}, or sizes beyond limits   */
    ATTN_ERR_MASK = -6,        /* bad mask_kind / pad_lens / causal value      */
    ATTN_ERR_ALIGN = -7,       /* a data pointer is not 16-byte aligned        */
    ATTN_ERR_LAUNCH = -8,      /* the HIP launch failed                        */
    ATTN_ERR_DEVICE = -9,      /* the current device is not gfx950             */
    ATTN_ERR_ALIAS = -10,      /* attn_fwd_rope: k_rot overlaps another tensor */
    ATTN_ERR_WORKSPACE = -11,  /* attn_fwd_decode: workspace too small         */
    ATTN_ERR_SCRATCH = -12     /* attn_fwd_decode_noalloc: sizes exceed its    *
                                * fixed workspace (32 MiB per GPU)              */
};

/*
 * attn_fwd — fused scaled-dot-product attention forward.
 *
 *   q, k, v     input descriptors (see above).  q: (B,S,Hq,D); k, v: (B,S,Hkv,D).
 *   mask_kind   ATTN_MASK_NONE or ATTN_MASK_KEY_PADDING.
 *   pad_lens    device int32[B] of valid key lengths when mask_kind is
 *               ATTN_MASK_KEY_PADDING (must be NULL otherwise).  Values are
 *               clamped to [0, S] on the device; a batch with length 0 has
 *               no visible key.
 *   scale       multiplier of Q·Kᵀ; any value that is not > 0 (0, negative,
 *               NaN) selects the default 1/sqrt(D) ("ops-transformer…" §4.2).
 *   causal      0 or 1; key j is visible to query i only if j <= i.  Causal
 *               and key padding compose (both must allow a key).
 *   n_q_heads   Hq (== q->H == out->H);  n_kv_heads  Hkv (== k->H == v->H),
 *               Hq % Hkv == 0; query head h reads kv head floor(h*Hkv/Hq).
 *   out         output descriptor: same B, S, D and dtype as q, H = Hq.
 *               A row with no visible key is written as zeros.
 *   lse         device float[B, Hq, S] receiving ln(sum_j exp(S_ij)) per row
 *               (-inf for a row with no visible key), or NULL to skip it.
 *   stream      hipStream_t to enqueue on (NULL = default stream).
 *
 * Limits: S < 2^29, Hq <= 65535, and one batch of K (or V) below 2 GiB:
 * S * n_kv_heads * D * sizeof(element) < 2^31 (ATTN_ERR_UNSUPPORTED).
 * Returns ATTN_OK or one of the negative codes above.
 */
int attn_fwd(const attn_tensor_t* q, const attn_tensor_t* k, const attn_tensor_t* v,
             int mask_kind, const int32_t* pad_lens, float scale, int causal,
             int n_q_heads, int n_kv_heads,
             const attn_tensor_t* out, float* lse, void* stream);

/*
 * attn_fwd_varlen — attn_fwd over packed sequences of different lengths.
 *
 * The ATB engineering guide (hwcomputing.csdn.net/6a59a88310ee7a33f28e5ce9)
 * §6.1 has the attention operator adapt at run time to sequence lengths that
 * vary per request (32 to 4096 tokens), and its §8.7 drives one MhaV3
 * operator over such lengths; "ops-transformer：Transformer算子融合与推理加速
 * 实战" §5.2 merges batch and heads into one parallel axis and then splits
 * the sequence.  Here a batch of such sequences is packed back to back with
 * no padding: sequence b is rows [cu_seqlens[b], cu_seqlens[b+1]) of
 *
 *   q, out: (1, T, Hq, D);  k, v: (1, T, Hkv, D)
 *
 * and each sequence is an independent self-attention over its own rows,
 * computed as attn_fwd documents (scale, GQA mapping, LSE definition), with
 * the causal rule counted within the sequence (key j visible to query i iff
 * j <= i, both counted from the sequence's first row).  No padded row is
 * computed and no padded key is read.
 *
 *   cu_seqlens  device int32[n_seqs + 1] (4-byte aligned), non-decreasing,
 *               within [0, T].  Offsets are clamped into [0, T] on the
 *               device (so a bad offset cannot leave the buffers).
 *   n_seqs      number of sequences B (>= 0).
 *   max_seqlen  an upper bound on every length, 0 <= max_seqlen <= T (else
 *               ATTN_ERR_SHAPE); it sizes the launch.  A longer sequence is
 *               treated as its first max_seqlen rows.
 *   out         rows inside a sequence are written; rows outside every
 *               sequence are left untouched.
 *   lse         device float[Hq, T] (row r of head h at h*T + r), or NULL.
 *   q, k, v, scale, causal, n_q_heads, n_kv_heads, stream: as for attn_fwd
 *               (descriptors with B == 1, S == T; else ATTN_ERR_SHAPE).
 *
 * Limits: as for attn_fwd with S = T.  n_seqs == 0, T == 0 or
 * max_seqlen == 0: ATTN_OK, nothing launched.  All checks precede the launch.
 */
int attn_fwd_varlen(const attn_tensor_t* q, const attn_tensor_t* k, const attn_tensor_t* v,
                    const int32_t* cu_seqlens, int n_seqs, int64_t max_seqlen, float scale, int causal,
                    int n_q_heads, int n_kv_heads, const attn_tensor_t* out, float* lse, void* stream);

/*
 * attn_fwd_masked — attn_fwd with an explicit additive mask tensor.
 *
 * The page "CANN-ATB图优化-昇腾NPU怎么把PyTorch计算图改造成融合算子" (Pattern 2)
 * fuses Q·Kᵀ → Scale → Mask → Softmax → ·V into FlashAttention(Q, K, V, mask,
 * scale), the mask entering after the scale; the ATB engineering guide
 * (hwcomputing.csdn.net/6a59a88310ee7a33f28e5ce9) §8.2 passes the mask to the
 * attention operator as one more FP16 input tensor.  Computed as attn_fwd
 * documents, with the scores
 *
 *   S_ij = (Q_i · K_j) · scale + M[b', h', i, j]
 *
 * where M is (mask_B, mask_H, S, S), contiguous, row-major, broadcast over
 * batch (mask_B == 1: b' = 0; mask_B == B: b' = b) and query heads (mask_H
 * == 1 or Hq).  -inf hides a key; a row whose every score is -inf is written
 * as zeros with LSE -inf.  causal (0/1) composes with the mask (j > i is
 * hidden as well).
 *
 *   mask        device pointer, 16-byte aligned (ATTN_ERR_ALIGN).
 *   mask_type   ATTN_MASK_ADDITIVE: M in q's dtype, values finite or -inf;
 *               ATTN_MASK_BOOL: one byte per entry, nonzero = the key takes
 *               part (M = 0), zero = hidden (M = -inf).  Else ATTN_ERR_MASK.
 *   mask_B      1 or q->B; mask_H  1 or n_q_heads (else ATTN_ERR_MASK).
 *   q, k, v, scale, causal, n_q_heads, n_kv_heads, out, lse, stream: as for
 *               attn_fwd (no key-padding argument: a mask expresses it).
 *
 * Supported: bf16 and fp16 (fp32 returns ATTN_ERR_UNSUPPORTED), D a
 * multiple of 16 in [16, 256], B <= 65535.  One launch; all checks precede it.
 */
int attn_fwd_masked(const attn_tensor_t* q, const attn_tensor_t* k, const attn_tensor_t* v,
                    const void* mask, int mask_type, int64_t mask_B, int64_t mask_H, float scale, int causal,
                    int n_q_heads, int n_kv_heads, const attn_tensor_t* out, float* lse, void* stream);

/*
 * attn_fwd_rope — rotary position embedding of Q and K fused with attn_fwd.
 *
 * The fifth fusion pattern of the ATB engineering guide
 * (hwcomputing.csdn.net/6a59a88310ee7a33f28e5ce9) §4.1 feeds RoPE(Q) and
 * RoPE(K) into the attention without materialising rotated tensors; its §8.4
 * configures the rotation (base 10000, interleaved pairs) and checks it
 * against a plain rotation of each (even, odd) dimension pair.  Computed:
 *
 *   theta_i = base^(-2i/D),  i = 0 .. D/2-1
 *   for Q and K, every head, row s of batch b at position p = positions[b,s]
 *   (or p = s when positions is NULL):
 *     x'[2i]   = x[2i]   cos(p theta_i) - x[2i+1] sin(p theta_i)
 *     x'[2i+1] = x[2i+1] cos(p theta_i) + x[2i]   sin(p theta_i)
 *   then attn_fwd(RoPE(Q), RoPE(K), V, ...) with every other argument as
 *   attn_fwd documents.  The rotated values are rounded to the input dtype
 *   before the products (as if RoPE ran as its own op); the angle is reduced
 *   in fp64, so any int32 position is accurate.
 *
 * Two launches on `stream`: a bandwidth-bound pass writes RoPE(K) into k_rot
 * (the form a KV cache keeps), then the attention kernel reads k_rot and
 * rotates each Q tile in registers as it loads it (Q is never written).
 *
 *   positions   device int32[B, S] (4-byte aligned) or NULL for 0 .. S-1;
 *               any int32 value is allowed.
 *   rope_base   rotary base; any value that is not > 0 and finite selects
 *               10000.
 *   k_rot       output descriptor with the shape and dtype of k, 16-byte
 *               aligned; receives RoPE(K).  It may be k itself (in-place
 *               rotation); any other overlap with k, q, v, out or lse returns
 *               ATTN_ERR_ALIAS.  Caller-owned like every other buffer.
 *
 * Returns ATTN_OK or a negative code; all checks run before any launch.
 */
int attn_fwd_rope(const attn_tensor_t* q, const attn_tensor_t* k, const attn_tensor_t* v,
                  int mask_kind, const int32_t* pad_lens, float scale, int causal,
                  int n_q_heads, int n_kv_heads, const int32_t* positions, float rope_base,
                  const attn_tensor_t* k_rot, const attn_tensor_t* out, float* lse, void* stream);

/*
 * attn_fwd_decode — decode attention over a KV cache (split over key chunks).
 *
 * The serving step the pages build around a KV cache: the ATB introduction
 * (hwcomputing.csdn.net/6a15a709662f9a54cb774da1) runs a causal
 * FlashAttention with KV-cache management on, and "CANN-ops-transformer和
 * ATB-昇腾NPU上算子和加速库怎么配合" has ATB pass the cache into and out of
 * FlashAttention on every generation step.  Computed, for every batch b,
 * query head h (kv head g = floor(h*Hkv/Hq)) and new row i < Sq:
 *
 *   L_b = cache_lens[b] clamped to [0, Sk]   (Sk when cache_lens is NULL)
 *   key j is visible iff j < L_b and, when causal, j <= L_b - Sq + i
 *     (the new rows are the last Sq positions of the sequence)
 *   O[b,i,h,:] = softmax_j(scale · q·k_j) · V,  LSE[b,h,i] = ln Σ_j exp(scale · q·k_j)
 *   (a row with no visible key: O = 0, LSE = -inf)
 *
 *   q, out      (B, Sq, Hq, D) descriptors; k_cache, v_cache (B, Sk, Hkv, D),
 *               Sk may differ from Sq; dtype and D as for attn_fwd.
 *   cache_lens  device int32[B] (4-byte aligned) or NULL.
 *   scale, causal, n_q_heads, n_kv_heads, lse, stream: as for attn_fwd
 *               (lse is (B, Hq, Sq)).
 *   workspace   caller-owned device buffer, 16-byte aligned, of at least
 *               attn_decode_workspace_bytes(B, Sq, Hq, D, Sk) bytes (else
 *               ATTN_ERR_WORKSPACE).  Its first 1024 bytes are arrival
 *               counters: they must be zero before the first call that uses
 *               the buffer (allocate it zero-filled, or clear it once), and
 *               every call leaves them zero again, so a buffer can serve any
 *               number of calls of any sizes it is large enough for.  The
 *               rest holds per-split partial results during a call and
 *               needs no initialisation.  Calls that share a workspace must
 *               not overlap (same stream, or otherwise ordered).
 *
 * Launches on `stream`: one workgroup per (split of the cache, batch, kv
 * head, 32 query rows; for fp32 256-key splits and 8 rows) writes the split's
 * partial (O, max, sums) to the workspace, and the splits are combined by
 * their log-sum-exp into O and LSE.  For bf16/fp16 the splits are as few as
 * fill the GPU (never more than the workspace was sized for); a call left
 * with one split writes O and LSE directly, and with up to 8 splits the last
 * split of each (batch, kv head, 32 query rows) to finish (counted in the
 * workspace's counters, which it returns to zero) merges them: one launch.
 * With more splits, and for fp32, a second kernel merges.
 * bf16/fp16 run both products on MFMA with fp32 accumulation, P rounded to
 * the input type, O normalised by the sum of the rounded probabilities and
 * LSE taken from the exact sum.
 * Limits: Sk < 2^29, Sq < 2^20, B·Hkv <= 65535.  Returns ATTN_OK (B == 0 or
 * Sq == 0: nothing launched) or a negative code; checks precede launches.
 */
int attn_fwd_decode(const attn_tensor_t* q, const attn_tensor_t* k_cache, const attn_tensor_t* v_cache,
                    const int32_t* cache_lens, float scale, int causal, int n_q_heads, int n_kv_heads,
                    const attn_tensor_t* out, float* lse, void* workspace, int64_t workspace_bytes,
                    void* stream);

/*
 * attn_fwd_decode_noalloc — attn_fwd_decode for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation.  Same arguments, checks, kernels and results as
 * attn_fwd_decode, minus the workspace: the per-chunk partial results go to a
 * fixed array inside the library, 32 MiB on each GPU it runs on, held until
 * the process ends.  Calls whose attn_decode_workspace_bytes(...) exceeds
 * 33554432 return ATTN_ERR_SCRATCH (before any HIP call).  The array's device
 * address is looked up (no allocation) on the first call on each device.
 *
 * Every call on one GPU shares that GPU's array.  Its arrival counters (the
 * first 1024 bytes, as in a caller workspace) are zero when the library is
 * loaded (a zero-initialised device array) and every call leaves them zero;
 * the partial results each call reads are ones it wrote itself, so nothing
 * needs clearing.  Calls that may overlap on one GPU (concurrent streams,
 * threads) race on the array: serialise them.  Nothing is allocated or freed
 * by this call.
 */
int attn_fwd_decode_noalloc(const attn_tensor_t* q, const attn_tensor_t* k_cache, const attn_tensor_t* v_cache,
                            const int32_t* cache_lens, float scale, int causal, int n_q_heads, int n_kv_heads,
                            const attn_tensor_t* out, float* lse, void* stream);

/* Bytes of workspace attn_fwd_decode needs for these sizes: 1024 bytes of
 * arrival counters, then one 256-key chunk (at least one, also for an empty
 * cache) × B·Hq·Sq rows × (D + 3) floats; -1 if a size is negative or the
 * count does not fit in int64. */
int64_t attn_decode_workspace_bytes(int64_t B, int64_t Sq, int n_q_heads, int64_t D, int64_t Sk);

/* Static, human-readable text for a return code (never NULL). */
const char* attn_strerror(int code);

/* Library version string, e.g. "attn_fwd 0.2.0 gfx950 src 0123456789abcdef":
 * the last word is the first 16 hex digits of the SHA-256 of the sources the
 * library was built from (static storage, never NULL). */
const char* attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_FWD_H */
