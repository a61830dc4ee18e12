"""attn_fwd_rope (rotary embedding of Q and K fused with the attention) vs
the fp64 oracle, through the C ABI.

Reference: oracle.rope on the rounded inputs, the rotated Q and K rounded to
the storage dtype (what an unfused rotation op would hand the attention),
then oracle.attention.  The rotated K the library writes (k_rot) is checked
element by element against the exact fp64 rotation: one rounding to the
storage dtype plus a small angle error; the ATB guide's own check of its RoPE
operator asks for max error < 1e-3 on fp16, which these bars are tighter than.
"""

import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import TORCH_DT, prep, to_np
from tolerances import assert_parity
from transformer_attention_06_amd import attn as A
from transformer_attention_06_amd import workloads as W

pytestmark = pytest.mark.gpu

# half an ulp (relative) of the storage dtype
HALF_ULP = {"bf16": 2.0 ** -8, "fp16": 2.0 ** -11, "fp32": 2.0 ** -24}


def _round(x, dtype):
    return torch.from_numpy(np.ascontiguousarray(x)).to(TORCH_DT[dtype]).to(torch.float64).numpy()


def _pair_norm(x):
    n = np.sqrt(x[..., 0::2] ** 2 + x[..., 1::2] ** 2)
    return np.repeat(n, 2, axis=-1)


def check_k_rot(k_rot, kn, kr_exact, dtype, what):
    """|k_rot - R(k)| <= half an ulp of R(k) + 2e-5 of the pair's length."""
    d = np.abs(np.asarray(k_rot, np.float64) - kr_exact)
    tol = HALF_ULP[dtype] * np.abs(kr_exact) + 2e-5 * _pair_norm(kn) + 1e-7
    bad = d > tol
    assert not bad.any(), f"{what}: k_rot err {d.max()} (worst at {np.argwhere(bad)[:3]})"
    return float(d.max())


def _run(seed, B, S, Hq, Hkv, D, dtype, *, causal=False, padded=False, positions=None, base=None,
         in_place=False, scale=None):
    q, k, v = W.random_inputs(seed, B, S, Hq, Hkv, D)
    pad = W.random_pad_lens(seed + 1, B, 0, S) if padded else None
    qd, qn = prep(q, dtype)
    kd, kn = prep(k, dtype)
    vd, vn = prep(v, dtype)
    pos_d = None if positions is None else torch.from_numpy(np.asarray(positions, np.int32)).cuda()
    pad_d = None if pad is None else torch.from_numpy(np.asarray(pad, np.int32)).cuda()
    out = torch.empty_like(qd)
    lse = torch.empty((B, Hq, S), dtype=torch.float32, device="cuda")
    k_rot = kd if in_place else torch.empty_like(kd)
    mk = A.ATTN_MASK_NONE if pad is None else A.ATTN_MASK_KEY_PADDING
    print(f"rope case seed={seed} B{B} S{S} H{Hq}/{Hkv} D{D} {dtype} causal={causal} padded={padded} "
          f"positions={'given' if positions is not None else 'default'} base={base} in_place={in_place}",
          flush=True)
    A.attn_fwd_rope(qd, kd, vd, mk, pad_d, scale, causal, Hq, Hkv, pos_d, base, k_rot, out, lse)
    torch.cuda.synchronize()
    b = oracle.ROPE_DEFAULT_BASE if base is None else base
    qr = oracle.rope(qn, positions, b)
    kr = oracle.rope(kn, positions, b)
    omk = oracle.MASK_NONE if pad is None else oracle.MASK_KEY_PADDING
    ro, rl = oracle.attention(_round(qr, dtype), _round(kr, dtype), vn, causal=causal, mask_kind=omk,
                              pad_lens=pad, scale=scale)
    return dict(out=to_np(out), lse=to_np(lse), k_rot=to_np(k_rot), ro=ro, rl=rl, kr=kr, kn=kn)


CASES = [
    # (seed, B, S, Hq, Hkv, D, dtype, causal, padded)
    (11, 1, 128, 2, 2, 64, "fp32", False, False),     # the tiny fp32 shape
    (12, 2, 200, 2, 2, 128, "fp32", True, False),
    (13, 1, 300, 4, 4, 128, "bf16", True, False),     # ragged: 2.3 query blocks
    (14, 2, 200, 6, 2, 64, "fp16", False, True),      # GQA + key padding
    (15, 1, 129, 8, 1, 128, "bf16", True, False),     # MQA, one row past a block
    (16, 2, 65, 4, 2, 128, "fp16", True, True),
    (17, 1, 64, 2, 2, 64, "bf16", False, False),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[6]}-D{c[5]}-S{c[2]}-H{c[3]}_{c[4]}-c{int(c[7])}p{int(c[8])}")
def test_rope_default_positions(case):
    seed, B, S, Hq, Hkv, D, dtype, causal, padded = case
    r = _run(seed, B, S, Hq, Hkv, D, dtype, causal=causal, padded=padded)
    check_k_rot(r["k_rot"], r["kn"], r["kr"], dtype, "k_rot")
    assert_parity(r["out"], r["ro"], dtype, lse=r["lse"], lse_ref=r["rl"], what=f"rope {case}")


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
def test_rope_given_positions(dtype):
    """Per-batch positions: far offsets (a decode-like cache position), repeats,
    negative values and the int32 extremes' neighbourhood."""
    B, S = 2, 150
    rng = np.random.default_rng(21)
    pos = np.empty((B, S), np.int64)
    pos[0] = 100000 + np.arange(S)
    pos[1] = rng.integers(-(2 ** 31) + 1, 2 ** 31 - 1, size=S)
    pos[1, :5] = [0, 0, -1, 2 ** 31 - 1, -(2 ** 31)]
    r = _run(22, B, S, 4, 2, 128 if dtype != "fp32" else 64, dtype, causal=True, positions=pos)
    check_k_rot(r["k_rot"], r["kn"], r["kr"], dtype, "k_rot (given positions)")
    assert_parity(r["out"], r["ro"], dtype, lse=r["lse"], lse_ref=r["rl"], what=f"positions {dtype}")


def test_rope_other_base_and_scale():
    r = _run(31, 1, 192, 4, 4, 128, "bf16", causal=True, base=500.0, scale=0.05)
    check_k_rot(r["k_rot"], r["kn"], r["kr"], "bf16", "k_rot base 500")
    assert_parity(r["out"], r["ro"], "bf16", lse=r["lse"], lse_ref=r["rl"], what="base 500")


def test_rope_in_place_matches_out_of_place():
    a = _run(41, 1, 160, 4, 2, 128, "bf16", causal=True)
    b = _run(41, 1, 160, 4, 2, 128, "bf16", causal=True, in_place=True)
    assert np.array_equal(a["k_rot"], b["k_rot"])
    assert np.array_equal(a["out"], b["out"])


def test_rope_position_zero_row_is_plain_attention_input():
    """Row 0 sits at position 0 (no rotation): its rotated K equals K."""
    r = _run(51, 1, 96, 2, 2, 64, "fp16")
    assert np.array_equal(r["k_rot"][:, 0], r["kn"][:, 0])


def test_rope_llama2_7b_prefill_shape():
    """The benchmark shape with the rotation: every element of k_rot, and
    sampled query rows of the output (first, block edges, diagonal, last)."""
    w = W.WORKLOADS["llama2_7b_prefill"]
    q, k, v, _ = W.make_inputs(w)
    qd, qn = prep(q, "bf16")
    kd, kn = prep(k, "bf16")
    vd, vn = prep(v, "bf16")
    print("rope case llama2_7b_prefill shape", flush=True)
    out, k_rot, lse = A.rope_attention(qd, kd, vd, causal=True, return_lse=True)
    torch.cuda.synchronize()
    kr = oracle.rope(kn)
    check_k_rot(to_np(k_rot), kn, kr, "bf16", "k_rot C2 shape")
    qr = _round(oracle.rope(qn), "bf16")
    krr = _round(kr, "bf16")
    rows = np.array([0, 1, 63, 64, 127, 128, 1023, 1024, 2046, 2047])
    o = to_np(out)
    l = to_np(lse)
    for h in (0, 13, 31):
        ro, rl = oracle.attention_rows(qr, krr, vn, 0, h, rows, causal=True)
        assert_parity(o[0, rows, h], ro, "bf16", lse=l[0, h, rows], lse_ref=rl, what=f"C2 rope head {h}")
