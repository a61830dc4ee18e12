"""Attention with an explicit additive mask tensor, in float64 (the oracle).

TEST INFRASTRUCTURE ONLY (see the package docstring): never used by the
product path.

What is computed, and where the pages fix it
--------------------------------------------
[graph-opt] Pattern 2 fuses the chain Q·Kᵀ, then Scale, then Mask, then
Softmax, then dropout, then ·V into FlashAttention(Q, K, V, mask, scale); the
mask is an operand of the fused call and is applied to the scaled scores.
[ATB-guide] §8.2 (its execute_mha wrapper) hands the attention mask to the
operator as one more FP16 input tensor of the mask's own shape, next to Q, K
and V.  Computed, for every batch b and query head h (kv head
g = floor(h · Hkv / Hq)):

    S_ij = (q_i · k_j) · scale + M[b', h', i, j]
    (and S_ij = -inf for j > i when causal is also set)
    P = softmax_j(S),  O_i = P · V,  LSE_i = ln Σ_j exp(S_ij)

with M of shape (Bm, Hm, S, S), Bm in {1, B} and Hm in {1, Hq} broadcast over
batch and heads (b' = b if Bm = B else 0, likewise h').

Readings (listed in the design doc): the mask is additive (a value of -inf hides
the key, 0 leaves it untouched, any finite value shifts the score), as the
pages' float mask tensor and the "Scale → Mask → Softmax" order imply; a
boolean mask (True: the key takes part, False: hidden) is the additive mask
with 0 and -inf; it is applied after the scale; causal masking composes with it; a row whose every
score is -inf has O = 0 and LSE = -inf; mask values are finite or -inf.
"""

import math

import numpy as np


def mask_slice(mask, b, h):
    """The (S, S) mask plane that batch b, query head h reads."""
    bm, hm = mask.shape[0], mask.shape[1]
    return mask[b if bm > 1 else 0, h if hm > 1 else 0]


def additive_from_bool(mask):
    """A boolean mask (True: the key takes part) as the additive mask it
    stands for: 0 where True, -inf where False."""
    mask = np.asarray(mask)
    return np.where(mask.astype(bool), 0.0, -np.inf)


def attention_masked(q, k, v, mask, *, causal=False, scale=None):
    """O (B, S, Hq, D) and LSE (B, Hq, S) under an additive mask (or a
    boolean one, read through additive_from_bool), float64."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    mask = np.asarray(mask)
    mask = additive_from_bool(mask) if mask.dtype == bool else mask.astype(np.float64)
    b_n, s, hq, d = q.shape
    hkv = k.shape[2]
    if k.shape[:2] != (b_n, s) or v.shape != k.shape or k.shape[3] != d:
        raise ValueError("q, k, v shapes disagree")
    if hq % hkv != 0:
        raise ValueError("query heads must be a multiple of kv heads")
    if mask.ndim != 4 or mask.shape[2:] != (s, s) or mask.shape[0] not in (1, b_n) or mask.shape[1] not in (1, hq):
        raise ValueError("mask must be (1 or B, 1 or Hq, S, S)")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = np.zeros((b_n, s, hq, d), dtype=np.float64)
    lse = np.full((b_n, hq, s), -np.inf, dtype=np.float64)
    above = np.triu(np.ones((s, s), dtype=bool), k=1)  # key j > query i
    for b in range(b_n):
        for h in range(hq):
            g = (h * hkv) // hq
            scores = (q[b, :, h, :] @ k[b, :, g, :].T) * scale + mask_slice(mask, b, h)
            if causal:
                scores = np.where(above, -np.inf, scores)
            m = scores.max(axis=1)
            has_key = np.isfinite(m)
            m_safe = np.where(has_key, m, 0.0)
            e = np.exp(scores - m_safe[:, None])
            den = e.sum(axis=1)
            safe = np.where(has_key, den, 1.0)
            out[b, :, h, :] = np.where(has_key[:, None], (e / safe[:, None]) @ v[b, :, g, :], 0.0)
            lse[b, h, :] = np.where(has_key, m_safe + np.log(safe), -np.inf)
    return out, lse
