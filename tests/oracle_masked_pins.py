"""Pins for the fp64 additive-mask oracle (oracle/masked.py).

Each ``pin_*`` takes the oracle module and raises AssertionError when its
``attention_masked`` disagrees with something that does not come from it:
the pinned prefill oracle (a zero mask; -inf above the diagonal standing in
for the causal flag; -inf past L_b standing in for key padding), torch's CPU
scaled_dot_product_attention in float64 with a float (additive) mask under
every broadcast shape (an independent library routine), the shift
invariance of the softmax (a per-row constant in the mask moves only LSE, by
exactly that constant), closed forms for fully masked rows, and a boolean
mask against both the hand-built additive one and torch's SDPA given the same
boolean mask.
"""

import math

import numpy as np


def _close(a, b, atol, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, (what, a.shape, b.shape)
    both_inf = np.isinf(a) & np.isinf(b) & (np.sign(a) == np.sign(b))
    # subtract only where the two are not the same infinity (inf - inf is NaN);
    # any other NaN difference counts as an infinite error
    d = np.subtract(a, b, out=np.zeros_like(a), where=~both_inf)
    err = np.abs(np.nan_to_num(d, nan=np.inf))
    assert np.all(err <= atol), f"{what}: max err {err.max()} at {np.argwhere(err > atol)[:3]}"


def _qkv(rng, b, s, hq, hkv, d):
    return (rng.standard_normal((b, s, hq, d)), rng.standard_normal((b, s, hkv, d)),
            rng.standard_normal((b, s, hkv, d)))


def pin_masked_zero_mask_is_plain(orc):
    """A zero mask changes nothing: equals the plain oracle, causal or not."""
    rng = np.random.default_rng(31)
    q, k, v = _qkv(rng, 2, 9, 4, 2, 8)
    for causal in (False, True):
        o, l = orc.attention_masked(q, k, v, np.zeros((1, 1, 9, 9)), causal=causal)
        po, pl = orc.attention(q, k, v, causal=causal)
        _close(o, po, 1e-12, f"O causal={causal}")
        _close(l, pl, 1e-12, f"LSE causal={causal}")


def pin_masked_triangle_is_causal(orc):
    """-inf above the diagonal (0 elsewhere) equals the causal flag."""
    rng = np.random.default_rng(32)
    q, k, v = _qkv(rng, 1, 12, 3, 3, 4)
    m = np.where(np.triu(np.ones((12, 12), bool), 1), -np.inf, 0.0)[None, None]
    o, l = orc.attention_masked(q, k, v, m)
    po, pl = orc.attention(q, k, v, causal=True)
    _close(o, po, 1e-12, "O")
    _close(l, pl, 1e-12, "LSE")


def pin_masked_key_padding(orc):
    """A per-batch mask (B, 1, S, S) with -inf on keys j >= L_b equals key
    padding, including a batch with L_b = 0 (every row fully masked)."""
    rng = np.random.default_rng(33)
    b, s = 3, 10
    q, k, v = _qkv(rng, b, s, 4, 1, 8)
    lens = np.array([10, 4, 0], np.int32)
    m = np.zeros((b, 1, s, s))
    for i, L in enumerate(lens):
        m[i, :, :, L:] = -np.inf
    for causal in (False, True):
        o, l = orc.attention_masked(q, k, v, m, causal=causal)
        po, pl = orc.attention(q, k, v, causal=causal, mask_kind=orc.MASK_KEY_PADDING, pad_lens=lens)
        _close(o, po, 1e-12, f"O causal={causal}")
        _close(l, pl, 1e-12, f"LSE causal={causal}")


def pin_masked_torch_sdpa(orc):
    """torch's CPU SDPA (float64, additive float mask, kv heads expanded) for
    every broadcast shape of the mask, with finite shifts and -inf holes; rows
    that keep at least one key."""
    import torch

    rng = np.random.default_rng(34)
    b, s, hq, hkv, d = 2, 11, 4, 2, 16
    q, k, v = _qkv(rng, b, s, hq, hkv, d)
    for shape in ((1, 1, s, s), (b, 1, s, s), (1, hq, s, s), (b, hq, s, s)):
        m = rng.standard_normal(shape) * 3.0
        m[rng.random(shape) < 0.3] = -np.inf
        m[..., 0] = 0.0  # key 0 always visible: no fully masked row here
        for causal, scale in ((False, None), (True, 0.37)):
            o, l = orc.attention_masked(q, k, v, m, causal=causal, scale=scale)
            sc = 1.0 / math.sqrt(d) if scale is None else scale
            tq = torch.from_numpy(q).permute(0, 2, 1, 3)
            tk = torch.from_numpy(k).permute(0, 2, 1, 3).repeat_interleave(hq // hkv, dim=1)
            tv = torch.from_numpy(v).permute(0, 2, 1, 3).repeat_interleave(hq // hkv, dim=1)
            tm = torch.from_numpy(m).expand(b, hq, s, s).clone()
            if causal:
                tm = tm.masked_fill(torch.ones(s, s, dtype=torch.bool).triu(1), float("-inf"))
            ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=tm, scale=sc)
            _close(o, ref.permute(0, 2, 1, 3).numpy(), 1e-12, f"O shape={shape} causal={causal}")
            # LSE from the same definition, by torch's logsumexp
            sco = torch.matmul(tq, tk.transpose(-1, -2)) * sc + tm
            _close(l, torch.logsumexp(sco, dim=-1).numpy(), 1e-12, f"LSE shape={shape} causal={causal}")


def pin_masked_row_shift(orc):
    """Adding a constant c_i to every entry of mask row i leaves O unchanged
    and adds exactly c_i to LSE_i (the mask enters unscaled, after the scale)."""
    rng = np.random.default_rng(35)
    q, k, v = _qkv(rng, 1, 8, 2, 2, 8)
    m = rng.standard_normal((1, 2, 8, 8))
    c = rng.uniform(-50.0, 50.0, size=(1, 2, 8, 1))
    for causal in (False, True):
        o, l = orc.attention_masked(q, k, v, m, causal=causal, scale=0.2)
        o2, l2 = orc.attention_masked(q, k, v, m + c, causal=causal, scale=0.2)
        _close(o2, o, 1e-12, f"O causal={causal}")
        _close(l2, l + c[..., 0], 1e-10, f"LSE causal={causal}")


def pin_masked_fully_masked_rows(orc):
    """Rows whose every key is -inf: O = 0, LSE = -inf, no NaN; other rows of
    the same head unaffected."""
    rng = np.random.default_rng(36)
    q, k, v = _qkv(rng, 1, 6, 2, 1, 4)
    m = np.zeros((1, 1, 6, 6))
    m[0, 0, 2, :] = -np.inf
    m[0, 0, 5, :] = -np.inf
    o, l = orc.attention_masked(q, k, v, m)
    assert np.all(o[0, [2, 5]] == 0.0) and np.all(np.isneginf(l[0, :, [2, 5]]))
    po, pl = orc.attention(q, k, v)
    keep = [0, 1, 3, 4]
    _close(o[0, keep], po[0, keep], 1e-12, "other rows")
    _close(l[0][:, keep], pl[0][:, keep], 1e-12, "other rows LSE")


def pin_masked_bool_mask(orc):
    """A boolean mask (True: the key takes part) equals the additive mask of
    zeros and -inf built by hand, and torch's CPU SDPA given the same boolean
    mask (its own convention: True takes part) in float64."""
    import torch

    rng = np.random.default_rng(37)
    b, s, hq, hkv, d = 2, 9, 4, 2, 8
    q, k, v = _qkv(rng, b, s, hq, hkv, d)
    bm = rng.random((b, 1, s, s)) < 0.7
    bm[..., 0] = True  # every row keeps a key
    add = np.zeros(bm.shape)
    add[~bm] = -np.inf
    for causal in (False, True):
        o, l = orc.attention_masked(q, k, v, bm, causal=causal)
        ao, al = orc.attention_masked(q, k, v, add, causal=causal)
        _close(o, ao, 0.0, f"O bool vs additive causal={causal}")
        _close(l, al, 0.0, f"LSE bool vs additive causal={causal}")
    tq = torch.from_numpy(q).permute(0, 2, 1, 3)
    tk = torch.from_numpy(k).permute(0, 2, 1, 3).repeat_interleave(hq // hkv, dim=1)
    tv = torch.from_numpy(v).permute(0, 2, 1, 3).repeat_interleave(hq // hkv, dim=1)
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=torch.from_numpy(bm))
    o, _ = orc.attention_masked(q, k, v, bm)
    _close(o, ref.permute(0, 2, 1, 3).numpy(), 1e-12, "O vs torch bool mask")


ALL_PINS = [
    pin_masked_zero_mask_is_plain,
    pin_masked_triangle_is_causal,
    pin_masked_key_padding,
    pin_masked_torch_sdpa,
    pin_masked_row_shift,
    pin_masked_fully_masked_rows,
    pin_masked_bool_mask,
]
