"""Attention over packed variable-length sequences in float64 (the oracle).

TEST INFRASTRUCTURE ONLY (see the package docstring): never used by the
product path.

What is computed, and where the pages fix it
--------------------------------------------
[ATB-guide] §6.1 says sequence lengths in serving are not fixed (a request
may be 32 tokens or 4096) and has the attention operator adapt to the actual
length at run time; its §8.7 drives one MhaV3 operator over lengths 32 to
4096.  [ops-transformer] §5.2 merges batch and heads into one parallel axis
and then splits the sequence.  A batch of such sequences is kept here packed
back to back, without padding: sequence b owns rows [cu[b], cu[b+1]) of

* q: (T, Hq, D); k, v: (T, Hkv, D)  (T rows in all, cu non-decreasing,
  cu[B] <= T);

and each sequence is an independent self-attention over its own rows, the
same scaled dot-product attention as the prefill oracle (oracle/attention.py):
scores (q_i · k_j) · scale, causal meaning key j is visible to query i iff
j <= i counted from the sequence's first row, a softmax over the visible keys,
the product with V, GQA head mapping floor(h · Hkv / Hq), scale defaulting to
1/sqrt(D), LSE the natural-log log-sum-exp of the scaled scores.

Readings (listed in the design doc): the packed layout with offsets cu[0..B] is
read as the batch form of the pages' dynamic lengths (no padding, no padded
rows computed); the causal rule is counted within each sequence (top-left);
LSE is laid out (Hq, T); rows outside every sequence are not part of the
output (returned here as O = 0, LSE = -inf, and never compared).
"""

import math

import numpy as np


def check_offsets(cu, total):
    """Validate the offsets: integers, non-decreasing, within [0, total]."""
    cu = np.asarray(cu, dtype=np.int64)
    if cu.ndim != 1 or cu.size < 1:
        raise ValueError("cu_seqlens must be a 1-D array of B+1 offsets")
    if np.any(np.diff(cu) < 0) or cu[0] < 0 or cu[-1] > total:
        raise ValueError("cu_seqlens must be non-decreasing within [0, T]")
    return cu


def attention_varlen(q, k, v, cu_seqlens, *, causal=False, scale=None):
    """O (T, Hq, D) and LSE (Hq, T) of every packed sequence, float64."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    t_n, hq, d = q.shape
    tk, hkv, dk = k.shape
    if tk != t_n or dk != d or v.shape != k.shape:
        raise ValueError("q, k, v shapes disagree")
    if hq % hkv != 0:
        raise ValueError("query heads must be a multiple of kv heads")
    cu = check_offsets(cu_seqlens, t_n)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = np.zeros((t_n, hq, d), dtype=np.float64)
    lse = np.full((hq, t_n), -np.inf, dtype=np.float64)
    for b in range(cu.size - 1):
        s0, s1 = int(cu[b]), int(cu[b + 1])
        n = s1 - s0
        if n == 0:
            continue
        # visible[i, j]: key j of this sequence for its query i (local indices)
        i_loc = np.arange(n)[:, None]
        j_loc = np.arange(n)[None, :]
        visible = (j_loc <= i_loc) if causal else np.ones((n, n), dtype=bool)
        for h in range(hq):
            g = (h * hkv) // hq
            scores = (q[s0:s1, h, :] @ k[s0:s1, g, :].T) * scale
            scores = np.where(visible, scores, -np.inf)
            m = scores.max(axis=1)
            e = np.exp(scores - m[:, None])
            den = e.sum(axis=1)
            out[s0:s1, h, :] = (e / den[:, None]) @ v[s0:s1, g, :]
            lse[h, s0:s1] = m + np.log(den)
    return out, lse
