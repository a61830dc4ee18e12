"""Plain scaled-dot-product attention in float64 (the oracle).

TEST INFRASTRUCTURE ONLY (see the package docstring): never used by the
product path.

What is computed, and where the pages fix it
--------------------------------------------
[graph-opt] "Pattern 2: SDPA -> FlashAttention" gives the operation chain the
fused kernel replaces: Q·Kᵀ, then scale, then mask, then softmax, then dropout,
then ·V.  [ATB-guide] §5.1 writes the same chain as a plain PyTorch function:
scores = (Q·Kᵀ)·scale, a softmax over the key axis, then a product with V.
[ops-transformer] §2.2 and §3.2 state that the blockwise online-softmax kernel
reaches that same result (it only reorganises the normalisation), so the
oracle is the plain definition with the whole S×S score matrix materialised.

Readings taken where the pages leave a step open (each is listed in the design doc):

* masked entries get probability exactly 0 (additive -inf);
* "padding mask with per-sequence valid lengths" masks KEYS j >= L_b for every
  query row of batch b; query rows past L_b are still computed;
* causal means key j is visible to query i iff j <= i (Sq == Sk here), and it
  composes with key padding by AND;
* a row with no visible key outputs O = 0 and LSE = -inf;
* GQA/MQA maps query head h to kv head floor(h * Hkv / Hq) (contiguous groups);
* dropout is the identity (inference forward);
* LSE is the natural-log log-sum-exp of the *scaled* scores, laid out
  (B, Hq, S);
* scale defaults to 1/sqrt(D) ([ops-transformer] §4.2; [ATB-guide] §5.1 and
  §8.2 both use 1/sqrt(head size)).

Arrays are (B, S, H, D) ([ops-transformer] §2.3 and §4.2 name this layout).
Inputs are whatever values the GPU reads (already rounded to the storage
dtype) given as float64.
"""

import math

import numpy as np

MASK_NONE = 0
MASK_KEY_PADDING = 1


def default_scale(d):
    """Scale used when none is given: 1/sqrt(D).

    [ops-transformer] §4.2: the scale coefficient defaults to one over the
    square root of D; leaving it out can cause numerical anomalies.
    """
    return 1.0 / math.sqrt(d)


def kv_head_for(h, n_q_heads, n_kv_heads):
    """K/V head read by query head ``h`` under MQA/GQA.

    [ATB-guide] §2.1 (MhaV2/MhaV3 support MQA/GQA) and §8.2 (head_num and a
    smaller kv_head_num) give only the head counts; the grouping is read as
    contiguous: query heads [g*G, (g+1)*G) share kv head g, G = Hq/Hkv.
    """
    if n_q_heads % n_kv_heads != 0:
        raise ValueError("n_q_heads must be a multiple of n_kv_heads")
    return (h * n_kv_heads) // n_q_heads


def allowed_keys(s, causal, key_len):
    """Boolean (S, S) matrix: entry [i, j] is True when query i may see key j.

    [graph-opt] Pattern 2 puts "Mask" between Scale and Softmax; [ATB-guide]
    §2.1 lists causal masking fused with the softmax, §8.2 sets is_causal.
    Causal: j <= i.  Key padding: j < key_len (key_len = S means no padding).
    """
    i = np.arange(s)[:, None]
    j = np.arange(s)[None, :]
    ok = j < key_len
    if causal:
        ok = ok & (j <= i)
    return np.broadcast_to(ok, (s, s)).copy()


def attention_head(qh, kh, vh, scale, causal=False, key_len=None):
    """One (batch, head): O (S, D) and natural-log LSE (S,), all float64.

    Steps in the order of [graph-opt] Pattern 2 (dropout = identity):
      1. scores = (Q·Kᵀ) · scale
      2. masked scores -> -inf
      3. softmax along keys with the row maximum subtracted first (the stable
         form; [ATB-guide] §7 names LogSumExp as the stable way to take the
         softmax's exponential sum)
      4. O = P · V;  LSE = m + ln(sum_j exp(s_ij - m))
    """
    qh = np.asarray(qh, dtype=np.float64)
    kh = np.asarray(kh, dtype=np.float64)
    vh = np.asarray(vh, dtype=np.float64)
    s_len = qh.shape[0]
    if key_len is None:
        key_len = s_len
    scores = (qh @ kh.T) * scale
    ok = allowed_keys(s_len, causal, key_len)
    scores = np.where(ok, scores, -np.inf)
    has_key = ok.any(axis=1)
    m = np.where(has_key, scores.max(axis=1, initial=-np.inf), 0.0)
    e = np.exp(scores - m[:, None])          # exp(-inf) = 0 for masked keys
    denom = e.sum(axis=1)
    safe = np.where(has_key, denom, 1.0)
    p = e / safe[:, None]
    out = p @ vh
    out[~has_key] = 0.0
    lse = np.where(has_key, m + np.log(safe), -np.inf)
    return out, lse


def _check_shapes(q, k, v, n_q_heads, n_kv_heads):
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("q, k, v must be (B, S, H, D)")
    b, s, hq, d = q.shape
    if k.shape != v.shape or k.shape[0] != b or k.shape[1] != s or k.shape[3] != d:
        raise ValueError("k, v must be (B, S, Hkv, D) matching q")
    if n_q_heads is None:
        n_q_heads = hq
    if n_kv_heads is None:
        n_kv_heads = k.shape[2]
    if hq != n_q_heads or k.shape[2] != n_kv_heads:
        raise ValueError("head counts disagree with the arrays")
    if n_q_heads % n_kv_heads != 0:
        raise ValueError("n_q_heads must be a multiple of n_kv_heads")
    return b, s, hq, d, n_q_heads, n_kv_heads


def _key_len(pad_lens, mask_kind, b, s):
    if mask_kind == MASK_NONE:
        return s
    if mask_kind != MASK_KEY_PADDING:
        raise ValueError("unknown mask_kind")
    return int(min(max(int(pad_lens[b]), 0), s))


def attention(q, k, v, *, causal=False, mask_kind=MASK_NONE, pad_lens=None,
              scale=None, n_q_heads=None, n_kv_heads=None):
    """Full attention forward: O (B, S, Hq, D) and LSE (B, Hq, S), float64.

    One (batch, head) at a time, as [ops-transformer] §3.2 describes the
    outer loops (batch and head are independent).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    b_n, s, hq, d, hq, hkv = _check_shapes(q, k, v, n_q_heads, n_kv_heads)
    if scale is None:
        scale = default_scale(d)
    out = np.zeros((b_n, s, hq, d), dtype=np.float64)
    lse = np.zeros((b_n, hq, s), dtype=np.float64)
    for b in range(b_n):
        key_len = _key_len(pad_lens, mask_kind, b, s)
        for h in range(hq):
            g = kv_head_for(h, hq, hkv)
            o_bh, l_bh = attention_head(q[b, :, h, :], k[b, :, g, :], v[b, :, g, :],
                                        scale, causal, key_len)
            out[b, :, h, :] = o_bh
            lse[b, h, :] = l_bh
    return out, lse


def attention_rows(q, k, v, b, h, rows, *, causal=False, mask_kind=MASK_NONE,
                   pad_lens=None, scale=None, n_q_heads=None, n_kv_heads=None):
    """Selected query rows of one (batch, head): O (R, D), LSE (R,), float64.

    The same definition as ``attention_head`` evaluated row by row, so that
    sampled outputs of very long sequences can be checked one at a time.
    """
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    b_n, s, hq, d, hq, hkv = _check_shapes(q, k, v, n_q_heads, n_kv_heads)
    if scale is None:
        scale = default_scale(d)
    key_len = _key_len(pad_lens, mask_kind, b, s)
    g = kv_head_for(h, hq, hkv)
    kh = np.asarray(k[b, :, g, :], dtype=np.float64)
    vh = np.asarray(v[b, :, g, :], dtype=np.float64)
    rows = np.asarray(rows, dtype=np.int64)
    out = np.zeros((len(rows), d), dtype=np.float64)
    lse = np.zeros(len(rows), dtype=np.float64)
    j = np.arange(s)
    for n, i in enumerate(rows):
        qi = np.asarray(q[b, i, h, :], dtype=np.float64)
        sc = (kh @ qi) * scale
        ok = j < key_len
        if causal:
            ok &= j <= i
        if not ok.any():
            out[n] = 0.0
            lse[n] = -np.inf
            continue
        sc = np.where(ok, sc, -np.inf)
        m = sc.max()
        e = np.exp(sc - m)
        den = e.sum()
        out[n] = (e / den) @ vh
        lse[n] = m + np.log(den)
    return out, lse
