"""Pins for the fp64 packed variable-length oracle (oracle/varlen.py).

Each ``pin_*`` takes the oracle module and raises AssertionError when its
``attention_varlen`` disagrees with something that does not come from it:
the pinned batched prefill oracle (equal lengths; key padding standing in
for a shorter sequence), torch's CPU scaled_dot_product_attention in float64
per sequence (an independent library routine), the closed form for uniform
scores (prefix means of V, LSE = ln(i+1)), and the independence of
sequences (changing one never moves another, empty sequences are no-ops).
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


def _packed(rng, lens, hq, hkv, d, extra=0):
    t = int(sum(lens)) + extra
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    q = rng.standard_normal((t, hq, d))
    k = rng.standard_normal((t, hkv, d))
    v = rng.standard_normal((t, hkv, d))
    return q, k, v, cu


def pin_varlen_equal_lengths_is_batched(orc):
    """B sequences of one length S packed back to back = the batched oracle
    on (B, S, H, D); LSE (Hq, B·S) = the batched (B, Hq, S) laid side by side."""
    rng = np.random.default_rng(11)
    for (b, s, hq, hkv, d, causal) in ((3, 5, 2, 2, 8, False), (2, 9, 4, 2, 4, True), (4, 3, 3, 1, 8, True)):
        q, k, v, cu = _packed(rng, [s] * b, hq, hkv, d)
        o, l = orc.attention_varlen(q, k, v, cu, causal=causal)
        bo, bl = orc.attention(q.reshape(b, s, hq, d), k.reshape(b, s, hkv, d), v.reshape(b, s, hkv, d),
                               causal=causal)
        _close(o, bo.reshape(b * s, hq, d), 1e-12, f"O b={b} s={s}")
        _close(l, bl.transpose(1, 0, 2).reshape(hq, b * s), 1e-12, f"LSE b={b} s={s}")


def pin_varlen_matches_key_padding(orc):
    """Sequence b of a packed batch = the first L_b rows of a padded batch
    whose keys past L_b are masked by the key-padding oracle (the padded rows
    hold unrelated values, which must never matter)."""
    rng = np.random.default_rng(12)
    lens = [5, 1, 8, 3]
    smax = 9
    hq, hkv, d = 4, 2, 8
    q, k, v, cu = _packed(rng, lens, hq, hkv, d)
    for causal in (False, True):
        o, l = orc.attention_varlen(q, k, v, cu, causal=causal)
        pq = rng.standard_normal((len(lens), smax, hq, d))
        pk = rng.standard_normal((len(lens), smax, hkv, d))
        pv = rng.standard_normal((len(lens), smax, hkv, d))
        for b, n in enumerate(lens):
            s0 = cu[b]
            pq[b, :n], pk[b, :n], pv[b, :n] = q[s0:s0 + n], k[s0:s0 + n], v[s0:s0 + n]
        po, pl = orc.attention(pq, pk, pv, causal=causal, mask_kind=orc.MASK_KEY_PADDING,
                               pad_lens=np.array(lens, np.int32))
        for b, n in enumerate(lens):
            s0 = cu[b]
            _close(o[s0:s0 + n], po[b, :n], 1e-12, f"O seq {b} causal={causal}")
            _close(l[:, s0:s0 + n], pl[b, :, :n], 1e-12, f"LSE seq {b} causal={causal}")


def pin_varlen_torch_sdpa(orc):
    """Per sequence, torch's CPU scaled_dot_product_attention in float64 with
    the kv heads expanded and an explicit scale (a library routine)."""
    import torch

    rng = np.random.default_rng(13)
    lens = [7, 0, 12, 1, 4]
    hq, hkv, d = 6, 2, 16
    q, k, v, cu = _packed(rng, lens, hq, hkv, d, extra=3)
    for causal, scale in ((False, None), (True, 0.3)):
        o, _ = orc.attention_varlen(q, k, v, cu, causal=causal, scale=scale)
        sc = 1.0 / math.sqrt(d) if scale is None else scale
        for b, n in enumerate(lens):
            if n == 0:
                continue
            s0 = cu[b]
            tq = torch.from_numpy(q[s0:s0 + n]).permute(1, 0, 2)
            tk = torch.from_numpy(k[s0:s0 + n]).permute(1, 0, 2).repeat_interleave(hq // hkv, dim=0)
            tv = torch.from_numpy(v[s0:s0 + n]).permute(1, 0, 2).repeat_interleave(hq // hkv, dim=0)
            ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=sc)
            _close(o[s0:s0 + n], ref.permute(1, 0, 2).numpy(), 1e-12, f"seq {b} causal={causal}")


def pin_varlen_uniform_scores(orc):
    """Q = 0: every visible score is 0, so row i of a sequence is the mean of
    its visible V rows (all n rows, or rows 0..i under causal masking) and
    LSE = ln(count)."""
    rng = np.random.default_rng(14)
    lens = [4, 6, 2]
    hq, hkv, d = 2, 1, 8
    _, k, v, cu = _packed(rng, lens, hq, hkv, d)
    q = np.zeros((int(cu[-1]), hq, d))
    for causal in (False, True):
        o, l = orc.attention_varlen(q, k, v, cu, causal=causal)
        for b, n in enumerate(lens):
            s0 = cu[b]
            for i in range(n):
                cnt = i + 1 if causal else n
                mean = v[s0:s0 + cnt, 0, :].mean(axis=0)
                for h in range(hq):
                    _close(o[s0 + i, h], mean, 1e-13, f"mean seq {b} row {i}")
                    _close(l[h, s0 + i], math.log(cnt), 1e-13, f"lse seq {b} row {i}")


def pin_varlen_sequences_independent(orc):
    """Changing one sequence's rows leaves every other sequence's output
    bit-identical and changes its own; an empty sequence inserted between
    two others changes nothing; rows outside every sequence are O = 0,
    LSE = -inf."""
    rng = np.random.default_rng(15)
    lens = [3, 5, 4]
    hq, hkv, d = 2, 2, 4
    q, k, v, cu = _packed(rng, lens, hq, hkv, d, extra=2)
    for causal in (False, True):
        o, l = orc.attention_varlen(q, k, v, cu, causal=causal)
        k2, v2 = k.copy(), v.copy()
        k2[cu[1]:cu[2]] += 3.0
        v2[cu[1]:cu[2]] -= 1.0
        o2, l2 = orc.attention_varlen(q, k2, v2, cu, causal=causal)
        for b in (0, 2):
            assert np.array_equal(o[cu[b]:cu[b + 1]], o2[cu[b]:cu[b + 1]]), f"seq {b} moved"
            assert np.array_equal(l[:, cu[b]:cu[b + 1]], l2[:, cu[b]:cu[b + 1]]), f"seq {b} LSE moved"
        assert not np.allclose(o[cu[1]:cu[2]], o2[cu[1]:cu[2]]), "changed sequence did not move"
        cu_e = np.array([cu[0], cu[1], cu[1], cu[2], cu[3]])
        oe, le = orc.attention_varlen(q, k, v, cu_e, causal=causal)
        assert np.array_equal(oe, o) and np.array_equal(le, l), "empty sequence changed the output"
        assert np.all(o[cu[-1]:] == 0.0) and np.all(np.isneginf(l[:, cu[-1]:])), "rows outside sequences"


def pin_varlen_rejects_bad_offsets(orc):
    """Offsets that decrease or leave [0, T] are rejected."""
    q = np.zeros((4, 1, 2))
    for cu in ([0, 3, 2], [0, 5], [-1, 2]):
        try:
            orc.attention_varlen(q, q, q, np.array(cu))
        except ValueError as e:
            assert "cu_seqlens" in str(e), f"offsets {cu} failed elsewhere: {e}"
            continue
        raise AssertionError(f"offsets {cu} accepted")


ALL_PINS = [
    pin_varlen_equal_lengths_is_batched,
    pin_varlen_matches_key_padding,
    pin_varlen_torch_sdpa,
    pin_varlen_uniform_scores,
    pin_varlen_sequences_independent,
    pin_varlen_rejects_bad_offsets,
]
