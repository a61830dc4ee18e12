"""Decode attention over a KV cache in float64 (the oracle).

TEST INFRASTRUCTURE ONLY (see the package docstring): never used by the
product path.

What is computed, and where the pages fix it
--------------------------------------------
The serving scenario the pages keep returning to is incremental decoding
over a KV cache: the ATB introduction (hwcomputing.csdn.net/
6a15a709662f9a54cb774da1) builds its graph operator from a causal
FlashAttention with KV-cache management switched on and a KVCache pool;
[ops+ATB] has ATB pass the cache into and out of FlashAttention on every
step; [ATB-guide] §6.2 asks LLaMA/GPT-style models to set num_kv_heads and
keep the cache in tiered storage; [ops-transformer] §5.1 has the bound of an
operator worked out from its bytes and FLOPs first, and at one query row per
sequence the cache bytes dominate.  A step attends Sq new query rows (usually
one per sequence) to the L_b cached keys and values of their sequence.  The arithmetic is the same scaled
dot-product attention as the prefill oracle (oracle/attention.py), with

* q: (B, Sq, Hq, D); the caches k, v: (B, Sk, Hkv, D) of which the first
  L_b = cache_lens[b] rows of batch b are valid (all Sk when not given);
* causal masking aligned to the END of the cache (the new rows are the last
  Sq positions): query row i of batch b sees key j iff j < L_b and
  j <= L_b - Sq + i.  Non-causal decoding sees every j < L_b;
* GQA head mapping, scale default, LSE definition and the empty-row rule
  (O = 0, LSE = -inf) exactly as in the prefill oracle.

Readings (listed in the design doc): the end-aligned causal rule is the one under
which a decode step over a cache equals the last Sq rows of a prefill over the
same sequence (pinned below); cache lengths are clamped to [0, Sk].
"""

import numpy as np

from .attention import default_scale, kv_head_for


def visible_keys(i, sq, key_len, causal):
    """Boolean mask over cache rows 0..key_len-1 for query row i (end-aligned)."""
    j = np.arange(key_len)
    if not causal:
        return np.ones(key_len, dtype=bool)
    return j <= key_len - sq + i


def attention_decode(q, k, v, *, cache_lens=None, causal=True, scale=None):
    """O (B, Sq, Hq, D) and LSE (B, Hq, Sq) of Sq query rows per sequence
    against the first cache_lens[b] rows of the caches, float64."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    b_n, sq, hq, d = q.shape
    kb, sk, hkv, kd = k.shape
    if kb != b_n or kd != d or v.shape != k.shape:
        raise ValueError("q, k, v shapes disagree")
    if scale is None:
        scale = default_scale(d)
    out = np.zeros((b_n, sq, hq, d), dtype=np.float64)
    lse = np.full((b_n, hq, sq), -np.inf, dtype=np.float64)
    for b in range(b_n):
        L = sk if cache_lens is None else int(min(max(int(cache_lens[b]), 0), sk))
        for h in range(hq):
            g = kv_head_for(h, hq, hkv)
            kh = k[b, :L, g, :]
            vh = v[b, :L, g, :]
            for i in range(sq):
                ok = visible_keys(i, sq, L, causal)
                if not ok.any():
                    continue
                s = (kh[ok] @ q[b, i, h, :]) * scale
                m = s.max()
                e = np.exp(s - m)
                den = e.sum()
                out[b, i, h, :] = (e / den) @ vh[ok]
                lse[b, h, i] = m + np.log(den)
    return out, lse
