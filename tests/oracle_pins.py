"""Pins for the fp64 oracle: facts fixed by the pages and the mathematics.

Each ``pin_*`` function takes the oracle module (``orc``) and raises
AssertionError when the oracle disagrees with something that does not come
from the oracle itself: a closed form, an invariant, an independent library
routine (torch's CPU scaled_dot_product_attention in float64), a
high-precision scalar brute force, or the hand-derived worked example in
``tests/golden/``.  ``tests/test_oracle_mutants.py`` runs every pin against
copies of the oracle with planted mistakes and requires each mistake to be
caught, so the set is known to be sharp.

Page short names as in the oracle package docstring.
"""

import json
import math
import os
from decimal import Decimal, getcontext

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _close(a, b, atol, rtol=0.0, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    if b.ndim == 0:
        b = np.broadcast_to(b, a.shape)
    assert a.shape == b.shape, (what, a.shape, b.shape)
    both_inf = np.isinf(a) & np.isinf(b) & (np.sign(a) == np.sign(b))
    with np.errstate(invalid="ignore"):
        err = np.where(both_inf, 0.0, np.abs(a - b))
    tol = atol + rtol * np.where(both_inf, 0.0, np.abs(b))
    bad = ~(err <= tol)
    assert not bad.any(), f"{what}: max err {np.nanmax(np.where(both_inf, 0, err))} at {np.argwhere(bad)[:3]}"


def _rng(seed):
    return np.random.default_rng(seed)


# --------------------------------------------------------------------------
# worked example (tests/golden/worked_example.json)
# --------------------------------------------------------------------------
def pin_worked_example(orc):
    """Hand-derived S=2, D=1 example; every value has a closed form."""
    with open(os.path.join(GOLDEN, "worked_example.json")) as f:
        g = json.load(f)
    for case in g["cases"]:
        q = np.array(case["q"], dtype=np.float64).reshape(1, 2, 1, 1)
        k = np.array(case["k"], dtype=np.float64).reshape(1, 2, 1, 1)
        v = np.array(case["v"], dtype=np.float64).reshape(1, 2, 1, 1)
        o, lse = orc.attention(q, k, v, causal=case["causal"])
        _close(o[0, :, 0, 0], case["out"], 1e-14, what=case["name"] + " out")
        _close(lse[0, 0, :], case["lse"], 1e-14, what=case["name"] + " lse")
        o2, l2 = orc.attention_rows(q, k, v, 0, 0, [0, 1], causal=case["causal"])
        _close(o2[:, 0], case["out"], 1e-14, what=case["name"] + " rows out")
        _close(l2, case["lse"], 1e-14, what=case["name"] + " rows lse")


# --------------------------------------------------------------------------
# closed forms of the fixed-pattern stress inputs
# ("ops-transformer：Transformer算子融合与推理加速实战" §4.2)
# --------------------------------------------------------------------------
def pin_stress_closed_forms(orc):
    with open(os.path.join(GOLDEN, "stress_closed_forms.json")) as f:
        g = json.load(f)
    for case in g["cases"]:
        b, s, h, d = case["shape"]
        x = np.full((b, s, h, d), case["fill"], dtype=np.float64)
        o, lse = orc.attention(x, x, x)
        _close(o, np.full_like(o, case["out"]), 0.0, what=case["name"] + " out")
        _close(lse, np.full_like(lse, case["lse"]), 1e-12, what=case["name"] + " lse")
        o2, l2 = orc.attention_rows(x, x, x, 0, 1, [0, s // 2, s - 1])
        _close(o2, np.full_like(o2, case["out"]), 0.0, what=case["name"] + " rows out")
        _close(l2, np.full_like(l2, case["lse"]), 1e-12, what=case["name"] + " rows lse")


def _n_allowed(s, causal, key_len):
    i = np.arange(s)
    n = np.full(s, key_len)
    if causal:
        n = np.minimum(i + 1, key_len)
    return n


def pin_uniform_scores_mean_of_v(orc):
    """Q = 0 makes every score equal: O_i is the mean of the visible V rows and
    LSE_i = ln(#visible keys); prefix means under causal masking, the first
    L_b rows under key padding, and O = 0 / LSE = -inf with no visible key."""
    rng = _rng(1)
    b_n, s, hq, hkv, d = 3, 9, 4, 2, 5
    q = np.zeros((b_n, s, hq, d))
    k = rng.standard_normal((b_n, s, hkv, d))
    v = rng.standard_normal((b_n, s, hkv, d))
    pad = np.array([9, 4, 0], dtype=np.int32)
    for causal in (False, True):
        for mk in (orc.MASK_NONE, orc.MASK_KEY_PADDING):
            o, lse = orc.attention(q, k, v, causal=causal, mask_kind=mk, pad_lens=pad)
            for b in range(b_n):
                kl = s if mk == orc.MASK_NONE else int(pad[b])
                n = _n_allowed(s, causal, kl)
                for h in range(hq):
                    g = h // (hq // hkv)
                    for i in range(s):
                        if n[i] == 0:
                            exp_o = np.zeros(d)
                            exp_l = -np.inf
                        else:
                            exp_o = v[b, : n[i], g, :].mean(axis=0)
                            exp_l = math.log(n[i])
                        _close(o[b, i, h], exp_o, 1e-13, what=f"mean b{b} h{h} i{i} c{causal} m{mk}")
                        _close(lse[b, h, i], exp_l, 1e-13, what=f"lse b{b} h{h} i{i}")
                    rows = list(range(s))
                    o2, l2 = orc.attention_rows(q, k, v, b, h, rows, causal=causal,
                                                mask_kind=mk, pad_lens=pad)
                    _close(o2, o[b, :, h], 1e-13, what="rows vs mean")
                    _close(l2, lse[b, h], 1e-13, what="rows lse vs mean")


def pin_one_hot_selection(orc):
    """Q_i = c·e_{pi(i)}, K_j = e_j: each row's score is c·scale on key pi(i)
    and 0 elsewhere.  With c·scale = 60 the softmax is one-hot to within
    e^-60, so O_i = V[pi(i)] and LSE_i = 60 + ln(1 + (n-1)e^-60).  pi is not
    an involution, so a transposed score matrix is caught."""
    s, d = 16, 64
    scale = 1.0 / math.sqrt(d)
    c = 60.0 / scale
    perm = np.roll(np.arange(s), 5)            # pi(i) = i - 5 mod 16
    q = np.zeros((1, s, 1, d))
    k = np.zeros((1, s, 1, d))
    for i in range(s):
        q[0, i, 0, perm[i]] = c
        k[0, i, 0, i] = 1.0
    v = _rng(2).standard_normal((1, s, 1, d))
    o, lse = orc.attention(q, k, v)
    _close(o[0, :, 0], v[0, perm, 0], 1e-20, what="one-hot out")
    _close(lse[0, 0], 60.0 + np.log1p((s - 1) * np.exp(-60.0)), 1e-12, what="one-hot lse")
    o2, l2 = orc.attention_rows(q, k, v, 0, 0, np.arange(s))
    _close(o2, v[0, perm, 0], 1e-20, what="one-hot rows")
    _close(l2, lse[0, 0], 1e-12, what="one-hot rows lse")
    # causal: rows with pi(i) > i cannot see their target; all their scores are 0
    oc, lc = orc.attention(q, k, v, causal=True)
    for i in range(s):
        if perm[i] <= i:
            _close(oc[0, i, 0], v[0, perm[i], 0], 1e-20, what=f"causal one-hot {i}")
            _close(lc[0, 0, i], 60.0 + np.log1p(i * np.exp(-60.0)), 1e-12)
        else:
            _close(oc[0, i, 0], v[0, : i + 1, 0].mean(axis=0), 1e-13, what=f"causal blind {i}")
            _close(lc[0, 0, i], math.log(i + 1), 1e-13)


def pin_rows_sum_to_one(orc):
    """V ≡ 1 gives O ≡ 1 for every row with a visible key (softmax rows sum to 1);
    a column-constant V gives that constant."""
    rng = _rng(3)
    b_n, s, hq, hkv, d = 2, 13, 6, 3, 4
    q = rng.standard_normal((b_n, s, hq, d)) * 3
    k = rng.standard_normal((b_n, s, hkv, d)) * 3
    cst = rng.standard_normal(d)
    v = np.broadcast_to(cst, (b_n, s, hkv, d)).copy()
    pad = np.array([13, 5], dtype=np.int32)
    for causal in (False, True):
        for mk in (orc.MASK_NONE, orc.MASK_KEY_PADDING):
            o, _ = orc.attention(q, k, v, causal=causal, mask_kind=mk, pad_lens=pad)
            _close(o, np.broadcast_to(cst, o.shape), 1e-13, what="column-constant V")


def pin_single_key(orc):
    """S = 1 ([ops-transformer] §6.4 single-element input): O = V[0],
    LSE = scale·q·k."""
    rng = _rng(4)
    for d in (1, 3, 64):
        q = rng.standard_normal((2, 1, 2, d))
        k = rng.standard_normal((2, 1, 1, d))
        v = rng.standard_normal((2, 1, 1, d))
        for causal in (False, True):
            o, lse = orc.attention(q, k, v, causal=causal)
            for b in range(2):
                for h in range(2):
                    _close(o[b, 0, h], v[b, 0, 0], 0.0, what="S=1 out")
                    _close(lse[b, h, 0], float(q[b, 0, h] @ k[b, 0, 0]) / math.sqrt(d), 1e-13)


def pin_first_causal_row(orc):
    """Under causal masking query 0 sees only key 0: O_0 = V[0], LSE_0 = scale·q0·k0."""
    rng = _rng(5)
    s, d = 33, 8
    q = rng.standard_normal((1, s, 3, d))
    k = rng.standard_normal((1, s, 3, d))
    v = rng.standard_normal((1, s, 3, d))
    o, lse = orc.attention(q, k, v, causal=True)
    for h in range(3):
        _close(o[0, 0, h], v[0, 0, h], 0.0, what="causal row 0")
        _close(lse[0, h, 0], float(q[0, 0, h] @ k[0, 0, h]) / math.sqrt(d), 1e-13)


def pin_scale_default(orc):
    """scale=None is 1/sqrt(D) ([ops-transformer] §4.2), bit for bit, and an
    explicit scale changes the result."""
    rng = _rng(6)
    q, k, v = (rng.standard_normal((1, 7, 2, 16)) for _ in range(3))
    a = orc.attention(q, k, v)
    b = orc.attention(q, k, v, scale=0.25)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    c = orc.attention(q, k, v, scale=1.0)
    assert not np.allclose(a[1], c[1])
    assert orc.default_scale(64) == 0.125


def pin_key_permutation(orc):
    """Without a mask, permuting K and V rows together changes nothing."""
    rng = _rng(7)
    s = 11
    q, k, v = (rng.standard_normal((2, s, 2, 6)) for _ in range(3))
    perm = rng.permutation(s)
    o1, l1 = orc.attention(q, k, v)
    o2, l2 = orc.attention(q, k[:, perm], v[:, perm])
    _close(o1, o2, 1e-13, what="perm out")
    _close(l1, l2, 1e-13, what="perm lse")


def pin_key_shift(orc):
    """K_j <- K_j + w for a fixed w shifts every score of row i by scale·q_i·w:
    O is unchanged and LSE_i grows by exactly that amount, even when the shift
    (here ~1e3 in score units) would overflow an unshifted exponential."""
    rng = _rng(8)
    s, d = 10, 8
    q = rng.standard_normal((1, s, 1, d))
    k = rng.standard_normal((1, s, 1, d))
    v = rng.standard_normal((1, s, 1, d))
    pad = np.array([7], dtype=np.int32)
    for scale_w in (0.5, 400.0):
        w = rng.standard_normal(d) * scale_w
        for causal in (False, True):
            for mk in (orc.MASK_NONE, orc.MASK_KEY_PADDING):
                o1, l1 = orc.attention(q, k, v, causal=causal, mask_kind=mk, pad_lens=pad)
                o2, l2 = orc.attention(q, k + w, v, causal=causal, mask_kind=mk, pad_lens=pad)
                shift = (q[0, :, 0] @ w) / math.sqrt(d)
                _close(o2, o1, 1e-9, what="shift out")
                _close(l2[0, 0], l1[0, 0] + shift, 1e-9, rtol=1e-12, what="shift lse")


def pin_gqa_mapping(orc):
    """Query head h reads kv head floor(h·Hkv/Hq) (contiguous groups).  With
    Q = 0 and V constant c_g on kv head g, O[..., h, :] = c_{g(h)}."""
    for hq, hkv in ((8, 2), (6, 3), (4, 1), (4, 4)):
        d, s = 3, 5
        q = np.zeros((1, s, hq, d))
        k = _rng(9).standard_normal((1, s, hkv, d))
        v = np.zeros((1, s, hkv, d))
        for g in range(hkv):
            v[0, :, g, :] = 10.0 * g + 1.0
        o, _ = orc.attention(q, k, v)
        grp = hq // hkv
        for h in range(hq):
            _close(o[0, :, h, :], np.full((s, d), 10.0 * (h // grp) + 1.0), 1e-13,
                   what=f"gqa h{h} of {hq}/{hkv}")
            o2, _ = orc.attention_rows(q, k, v, 0, h, [0, s - 1])
            _close(o2, np.full((2, d), 10.0 * (h // grp) + 1.0), 1e-13, what="gqa rows")


def pin_gqa_equals_expanded_mha(orc):
    rng = _rng(10)
    hq, hkv = 6, 2
    q = rng.standard_normal((2, 9, hq, 4))
    k = rng.standard_normal((2, 9, hkv, 4))
    v = rng.standard_normal((2, 9, hkv, 4))
    ke = np.repeat(k, hq // hkv, axis=2)
    ve = np.repeat(v, hq // hkv, axis=2)
    for causal in (False, True):
        o1, l1 = orc.attention(q, k, v, causal=causal)
        o2, l2 = orc.attention(q, ke, ve, causal=causal)
        _close(o1, o2, 1e-13, what="gqa vs expanded")
        _close(l1, l2, 1e-13, what="gqa lse vs expanded")


def pin_padding_is_truncation(orc):
    """Key padding with valid length L equals attention over K[:L], V[:L] only."""
    rng = _rng(11)
    s, d = 12, 5
    q, k, v = (rng.standard_normal((3, s, 2, d)) for _ in range(3))
    pad = np.array([12, 7, 1], dtype=np.int32)
    for causal in (False, True):
        o, lse = orc.attention(q, k, v, causal=causal, mask_kind=orc.MASK_KEY_PADDING, pad_lens=pad)
        for b in range(3):
            L = int(pad[b])
            qt = q[b:b + 1, :L]
            ot, lt = orc.attention(qt, k[b:b + 1, :L], v[b:b + 1, :L], causal=causal)
            _close(o[b, :L], ot[0], 1e-13, what=f"pad b{b} rows<L")
            _close(lse[b, :, :L], lt[0], 1e-13, what=f"pad lse b{b}")
            # rows past L see all L valid keys (causal or not): the same query
            # repeated at every position of an unmasked length-L problem
            for i in range(L, s):
                rows_q = np.repeat(q[b:b + 1, i:i + 1], L, axis=1)
                orow, lrow = orc.attention(rows_q, k[b:b + 1, :L], v[b:b + 1, :L])
                _close(o[b, i], orow[0, 0], 1e-13, what=f"pad past-L row {i}")
                _close(lse[b, :, i], lrow[0, :, 0], 1e-13, what=f"pad past-L lse {i}")


def pin_fully_masked_rows(orc):
    """Valid length 0: no row sees a key, O = 0 and LSE = -inf, no NaN."""
    rng = _rng(12)
    q, k, v = (rng.standard_normal((2, 6, 1, 3)) for _ in range(3))
    pad = np.array([0, 3], dtype=np.int32)
    for causal in (False, True):
        o, lse = orc.attention(q, k, v, causal=causal, mask_kind=orc.MASK_KEY_PADDING, pad_lens=pad)
        assert np.all(o[0] == 0.0) and np.all(np.isneginf(lse[0]))
        assert np.all(np.isfinite(o[1])) and np.all(np.isfinite(lse[1]))
        o2, l2 = orc.attention_rows(q, k, v, 0, 0, range(6), causal=causal,
                                    mask_kind=orc.MASK_KEY_PADDING, pad_lens=pad)
        assert np.all(o2 == 0.0) and np.all(np.isneginf(l2))


# --------------------------------------------------------------------------
# an independent library routine: torch's CPU SDPA in float64
# --------------------------------------------------------------------------
def pin_torch_sdpa(orc):
    import torch
    import torch.nn.functional as F
    rng = _rng(13)
    cases = [
        (1, 17, 2, 2, 8), (2, 33, 4, 2, 16), (3, 64, 8, 1, 64), (2, 50, 6, 3, 128), (1, 5, 3, 3, 1),
    ]
    for (b_n, s, hq, hkv, d) in cases:
        q = rng.standard_normal((b_n, s, hq, d)) * 2
        k = rng.standard_normal((b_n, s, hkv, d)) * 2
        v = rng.standard_normal((b_n, s, hkv, d))
        pad = rng.integers(1, s, size=b_n, endpoint=True).astype(np.int32)
        for causal in (False, True):
            for mk in (orc.MASK_NONE, orc.MASK_KEY_PADDING):
                for scale in (None, 0.3):
                    o, _ = orc.attention(q, k, v, causal=causal, mask_kind=mk, pad_lens=pad,
                                         scale=scale)
                    tq = torch.from_numpy(q).permute(0, 2, 1, 3)
                    tk = torch.from_numpy(k).permute(0, 2, 1, 3)
                    tv = torch.from_numpy(v).permute(0, 2, 1, 3)
                    mask = torch.ones(b_n, 1, s, s, dtype=torch.bool)
                    if causal:
                        mask &= torch.ones(s, s, dtype=torch.bool).tril()
                    if mk == orc.MASK_KEY_PADDING:
                        keyok = torch.arange(s)[None, :] < torch.from_numpy(pad).long()[:, None]
                        mask &= keyok[:, None, None, :]
                    ref = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, scale=scale,
                                                         enable_gqa=(hq != hkv))
                    ref = ref.permute(0, 2, 1, 3).numpy()
                    _close(o, ref, 1e-12, rtol=1e-12, what=f"sdpa {b_n,s,hq,hkv,d} c{causal} m{mk}")
                    rows = [0, s // 2, s - 1]
                    for hsel in range(hq):
                        o2, _ = orc.attention_rows(q, k, v, b_n - 1, hsel, rows, causal=causal,
                                                   mask_kind=mk, pad_lens=pad, scale=scale)
                        _close(o2, ref[b_n - 1, rows, hsel], 1e-12, rtol=1e-12,
                               what=f"sdpa rows h{hsel}")


# --------------------------------------------------------------------------
# high-precision scalar brute force on tiny inputs
# --------------------------------------------------------------------------
def _decimal_attention(q, k, v, causal, key_lens, scale, hq, hkv):
    getcontext().prec = 50
    b_n, s, _, d = q.shape
    sc = Decimal(repr(float(scale)))
    out = np.zeros((b_n, s, hq, d))
    lse = np.zeros((b_n, hq, s))
    for b in range(b_n):
        for h in range(hq):
            g = h // (hq // hkv)
            for i in range(s):
                js = [j for j in range(s) if j < key_lens[b] and (not causal or j <= i)]
                if not js:
                    out[b, i, h] = 0.0
                    lse[b, h, i] = -np.inf
                    continue
                scores = []
                for j in js:
                    acc = Decimal(0)
                    for t in range(d):
                        acc += Decimal(float(q[b, i, h, t])) * Decimal(float(k[b, j, g, t]))
                    scores.append(acc * sc)
                tot = sum((x.exp() for x in scores), Decimal(0))
                for t in range(d):
                    num = sum((x.exp() * Decimal(float(v[b, j, g, t])) for x, j in zip(scores, js)),
                              Decimal(0))
                    out[b, i, h, t] = float(num / tot)
                lse[b, h, i] = float(tot.ln())
    return out, lse


def pin_decimal_brute_force(orc):
    rng = _rng(14)
    for (b_n, s, hq, hkv, d) in ((1, 1, 1, 1, 1), (2, 3, 2, 1, 2), (1, 4, 4, 2, 4),
                                 (2, 7, 2, 2, 3), (1, 8, 2, 1, 4)):
        q = rng.standard_normal((b_n, s, hq, d)) * 2
        k = rng.standard_normal((b_n, s, hkv, d)) * 2
        v = rng.standard_normal((b_n, s, hkv, d))
        scale = 1.0 / math.sqrt(d)
        for causal in (False, True):
            for pad in (None, rng.integers(0, s, size=b_n, endpoint=True).astype(np.int32)):
                mk = orc.MASK_NONE if pad is None else orc.MASK_KEY_PADDING
                kl = [s] * b_n if pad is None else [int(x) for x in pad]
                o, lse = orc.attention(q, k, v, causal=causal, mask_kind=mk, pad_lens=pad)
                od, ld = _decimal_attention(q, k, v, causal, kl, scale, hq, hkv)
                _close(o, od, 1e-13, rtol=1e-12, what=f"decimal out {b_n,s,hq,hkv,d}")
                _close(lse, ld, 1e-13, rtol=1e-12, what=f"decimal lse {b_n,s,hq,hkv,d}")


ALL_PINS = [
    pin_worked_example,
    pin_stress_closed_forms,
    pin_uniform_scores_mean_of_v,
    pin_one_hot_selection,
    pin_rows_sum_to_one,
    pin_single_key,
    pin_first_causal_row,
    pin_scale_default,
    pin_key_permutation,
    pin_key_shift,
    pin_gqa_mapping,
    pin_gqa_equals_expanded_mha,
    pin_padding_is_truncation,
    pin_fully_masked_rows,
    pin_torch_sdpa,
    pin_decimal_brute_force,
]
