"""Pins for the fp64 decode oracle (oracle/decode.py).

Each ``pin_*`` takes the oracle module and raises AssertionError when its
``attention_decode`` disagrees with something that does not come from it:
the pinned prefill oracle on the same sequence (a decode step over a cache
equals the last rows of a prefill), a perturbation of cache rows past the
valid length, the merge of two key halves by their log-sum-exp (the rule a
split-KV kernel relies on), torch's CPU scaled_dot_product_attention in
float64 (an independent library routine, given an explicit boolean mask),
and closed forms for rows that see no key.
"""

import math

import numpy as np


def _close(a, b, atol, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, (what, a.shape, b.shape)
    both_inf = np.isinf(a) & np.isinf(b) & (np.sign(a) == np.sign(b))
    err = np.where(both_inf, 0.0, np.abs(np.nan_to_num(a - b, nan=np.inf)))
    assert np.all(err <= atol), f"{what}: max err {err.max()} at {np.argwhere(err > atol)[:3]}"


def _rng(seed):
    return np.random.default_rng(seed)


def pin_decode_equals_prefill_tail(orc):
    """Sq new rows against a cache of L rows = the last Sq rows of a causal
    prefill over the same L-token sequence (end-aligned causal rule)."""
    rng = _rng(1)
    for (L, sq, hq, hkv, d) in ((9, 1, 2, 2, 8), (12, 3, 4, 2, 8), (7, 7, 2, 1, 4), (20, 5, 6, 3, 16)):
        q = rng.standard_normal((2, L, hq, d))
        k = rng.standard_normal((2, L, hkv, d))
        v = rng.standard_normal((2, L, hkv, d))
        po, pl = orc.attention(q, k, v, causal=True)
        do, dl = orc.attention_decode(q[:, L - sq:], k, v, causal=True)
        _close(do, po[:, L - sq:], 1e-12, f"O L={L} sq={sq}")
        _close(dl, pl[:, :, L - sq:], 1e-12, f"LSE L={L} sq={sq}")


def pin_decode_cache_lengths(orc):
    """Rows of the cache at or past L_b never matter; L_b = Sk is the default;
    a per-batch L_b equals slicing that batch's cache."""
    rng = _rng(2)
    b, sq, sk, hq, hkv, d = 3, 2, 16, 4, 2, 8
    q = rng.standard_normal((b, sq, hq, d))
    k = rng.standard_normal((b, sk, hkv, d))
    v = rng.standard_normal((b, sk, hkv, d))
    lens = np.array([5, 16, 11])
    o1, l1 = orc.attention_decode(q, k, v, cache_lens=lens)
    k2, v2 = k.copy(), v.copy()
    for bb, L in enumerate(lens):
        k2[bb, L:] = 1e3 * rng.standard_normal((sk - L, hkv, d))
        v2[bb, L:] = -7.0
    o2, l2 = orc.attention_decode(q, k2, v2, cache_lens=lens)
    _close(o2, o1, 0.0, "rows past L_b")
    _close(l2, l1, 0.0, "rows past L_b (LSE)")
    for bb, L in enumerate(lens):
        os_, ls_ = orc.attention_decode(q[bb:bb + 1], k[bb:bb + 1, :L], v[bb:bb + 1, :L])
        _close(o1[bb:bb + 1], os_, 1e-13, f"batch {bb} sliced")
        _close(l1[bb:bb + 1], ls_, 1e-13, f"batch {bb} sliced (LSE)")
    od, ld = orc.attention_decode(q, k, v)
    of, lf = orc.attention_decode(q, k, v, cache_lens=np.full(b, sk))
    _close(od, of, 0.0, "default lengths")


def pin_decode_split_merge(orc):
    """Splitting the keys into [0, c) and [c, L) (non-causal, one row) and
    merging the two partial results by their LSE gives the whole result:
    O = sum_s exp(lse_s - lse) O_s, lse = log sum_s exp(lse_s)."""
    rng = _rng(3)
    L, hq, hkv, d = 37, 2, 1, 8
    q = rng.standard_normal((1, 1, hq, d)) * 2
    k = rng.standard_normal((1, L, hkv, d))
    v = rng.standard_normal((1, L, hkv, d))
    o, l = orc.attention_decode(q, k, v, causal=False)
    for c in (1, 10, 36):
        o1, l1 = orc.attention_decode(q, k[:, :c], v[:, :c], causal=False)
        o2, l2 = orc.attention_decode(q, k[:, c:], v[:, c:], causal=False)
        for h in range(hq):
            a, bb = l1[0, h, 0], l2[0, h, 0]
            m = max(a, bb)
            lse = m + math.log(math.exp(a - m) + math.exp(bb - m))
            om = math.exp(a - lse) * o1[0, 0, h] + math.exp(bb - lse) * o2[0, 0, h]
            _close(om, o[0, 0, h], 1e-12, f"merged O split {c}")
            _close(lse, l[0, h, 0], 1e-12, f"merged LSE split {c}")


def pin_decode_torch_sdpa(orc):
    """torch's CPU scaled_dot_product_attention in float64 with an explicit
    end-aligned boolean mask (repeated kv heads for GQA)."""
    import torch
    rng = _rng(4)
    for (b, sq, sk, hq, hkv, d, causal) in ((2, 3, 19, 4, 2, 16, True), (1, 1, 40, 8, 1, 8, True),
                                           (2, 4, 9, 2, 2, 8, False)):
        q = rng.standard_normal((b, sq, hq, d))
        k = rng.standard_normal((b, sk, hkv, d))
        v = rng.standard_normal((b, sk, hkv, d))
        lens = rng.integers(sq, sk + 1, size=b)
        o, _ = orc.attention_decode(q, k, v, cache_lens=lens, causal=causal, scale=0.3)
        rep = hq // hkv
        for bb in range(b):
            L = int(lens[bb])
            qt = torch.from_numpy(q[bb]).permute(1, 0, 2)                       # (hq, sq, d)
            kt = torch.from_numpy(k[bb, :L]).permute(1, 0, 2).repeat_interleave(rep, 0)
            vt = torch.from_numpy(v[bb, :L]).permute(1, 0, 2).repeat_interleave(rep, 0)
            i = torch.arange(sq)[:, None]
            j = torch.arange(L)[None, :]
            mask = (j <= L - sq + i) if causal else torch.ones(sq, L, dtype=torch.bool)
            ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=0.3)
            _close(o[bb], ref.permute(1, 0, 2).numpy(), 1e-12, f"sdpa b{bb} causal={causal}")


def pin_decode_rows_without_keys(orc):
    """L_b < Sq under the causal rule: row i sees keys j <= L_b - Sq + i, so
    the first Sq - L_b rows see none (O = 0, LSE = -inf); L_b = 0 empties all."""
    rng = _rng(5)
    q = rng.standard_normal((2, 4, 2, 8))
    k = rng.standard_normal((2, 6, 2, 8))
    v = rng.standard_normal((2, 6, 2, 8))
    o, l = orc.attention_decode(q, k, v, cache_lens=np.array([2, 0]))
    _close(o[0, :2], np.zeros((2, 2, 8)), 0.0, "rows 0, 1 of batch 0")
    assert np.all(np.isneginf(l[0, :, :2])) and np.all(np.isfinite(l[0, :, 2:]))
    _close(o[0, 2], np.asarray(v[0, 0]), 1e-12, "row 2 sees only key 0")   # one visible key
    _close(l[0, :, 2], (k[0, 0] * q[0, 2]).sum(-1) / math.sqrt(8), 1e-12, "LSE of one key = its score")
    _close(o[1], np.zeros((4, 2, 8)), 0.0, "empty cache")
    assert np.all(np.isneginf(l[1]))


ALL_PINS = [
    pin_decode_equals_prefill_tail,
    pin_decode_cache_lengths,
    pin_decode_split_merge,
    pin_decode_torch_sdpa,
    pin_decode_rows_without_keys,
]
