"""attn_fwd_varlen (packed sequences of different lengths) vs the fp64 packed
oracle, through the C ABI.

Cases cover lengths at and around the 128-row query block and 64-key tile
(0, 1, 63, 64, 127, 128, 129, ...), empty sequences, offsets that do not start
at row 0, rows outside every sequence (which must stay untouched), a launch
bound larger than the longest sequence, GQA/MQA, causal and not, every dtype
and head dimension, bit equality with attn_fwd when all lengths are equal,
and the batched short-sequence shape (16 sequences of 128..512 rows, 32
heads, D = 64, fp16) at full size.
"""

import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import TORCH_DT, prep, to_np
from tolerances import assert_parity
from transformer_attention_06_amd import attn as A

pytestmark = pytest.mark.gpu

SENTINEL = 7.0


def _inputs(seed, total, hq, hkv, d, dtype):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((total, hq, d)).astype(np.float32)
    k = rng.standard_normal((total, hkv, d)).astype(np.float32)
    v = rng.standard_normal((total, hkv, d)).astype(np.float32)
    qd, qn = prep(q, dtype)
    kd, kn = prep(k, dtype)
    vd, vn = prep(v, dtype)
    return (qd, kd, vd), (qn, kn, vn)


def _run(dev, cu, max_len, causal, scale=None):
    qd, kd, vd = dev
    hq, hkv = qd.shape[1], kd.shape[1]
    out = torch.full_like(qd, SENTINEL)
    lse = torch.full((hq, qd.shape[0]), SENTINEL, dtype=torch.float32, device=qd.device)
    cu_d = torch.from_numpy(np.asarray(cu, np.int32)).cuda()
    A.attn_fwd_varlen(qd, kd, vd, cu_d, max_len, scale, causal, hq, hkv, out, lse)
    torch.cuda.synchronize()
    return to_np(out), lse.cpu().numpy()


def _check(seed, lens, hq, hkv, d, dtype, causal, *, start=0, tail=0, max_extra=0, scale=None):
    cu = np.concatenate([[start], start + np.cumsum(lens)]).astype(np.int64)
    total = int(cu[-1]) + tail
    max_len = min(max(lens) + max_extra, total) if len(lens) else 0
    print(f"varlen case seed={seed} lens={list(lens)} start={start} tail={tail} H{hq}/{hkv} D{d} {dtype} "
          f"causal={causal} max_len={max_len}", flush=True)
    dev, host = _inputs(seed, total, hq, hkv, d, dtype)
    o, l = _run(dev, cu, max_len, causal, scale)
    ro, rl = oracle.attention_varlen(*host, cu, causal=causal, scale=scale)
    inside = np.zeros(total, bool)
    inside[cu[0]:cu[-1]] = True
    assert np.all(o[~inside] == SENTINEL) and np.all(l[:, ~inside] == SENTINEL), "rows outside were written"
    if inside.any():
        assert_parity(o[inside], ro[inside], dtype, lse=l[:, inside], lse_ref=rl[:, inside],
                      what=f"varlen {lens}")


CASES = [
    # seed, lens, Hq, Hkv, D, dtype, causal
    (1, [0, 1, 63, 64, 127, 128, 129, 300, 513], 4, 2, 128, "bf16", True),
    (2, [0, 1, 63, 64, 127, 128, 129, 300, 513], 4, 2, 128, "bf16", False),
    (3, [200, 5, 0, 0, 384, 257], 8, 1, 64, "fp16", True),
    (4, [200, 5, 0, 0, 384, 257], 8, 8, 64, "fp16", False),
    (5, [33, 256, 100], 2, 1, 128, "fp32", True),
    (6, [130, 1, 64], 3, 3, 64, "fp32", False),
    (7, [1000, 17], 6, 2, 128, "fp16", True),
    (8, [640], 2, 2, 64, "bf16", True),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[5]}-D{c[4]}-c{int(c[6])}-{len(c[1])}seq")
def test_varlen(case):
    seed, lens, hq, hkv, d, dtype, causal = case
    _check(seed, lens, hq, hkv, d, dtype, causal)


def test_varlen_offsets_not_at_zero_and_tail_rows():
    """Sequences starting at row 17, 9 rows after the last one: only the
    sequences' rows are written; a launch bound above the longest length."""
    _check(11, [129, 40, 0, 250], 4, 1, 128, "bf16", True, start=17, tail=9, max_extra=70)
    _check(12, [129, 40, 0, 250], 4, 2, 64, "fp16", False, start=3, tail=1, max_extra=5, scale=0.05)


def test_varlen_all_empty():
    _check(13, [0, 0, 0], 2, 1, 64, "bf16", True, tail=12)


@pytest.mark.parametrize("dtype,d,causal", [("bf16", 128, True), ("fp16", 64, False), ("fp32", 64, True)])
def test_varlen_equal_lengths_bitwise_equal_to_batched(dtype, d, causal):
    """Equal lengths packed back to back run the same tiles as attn_fwd over
    (B, S, H, D): outputs and LSE must be bit-identical."""
    b, s, hq, hkv = 3, 300, 4, 2
    rng = np.random.default_rng(21)
    q = torch.from_numpy(rng.standard_normal((b, s, hq, d)).astype(np.float32)).to(TORCH_DT[dtype]).cuda()
    k = torch.from_numpy(rng.standard_normal((b, s, hkv, d)).astype(np.float32)).to(TORCH_DT[dtype]).cuda()
    v = torch.from_numpy(rng.standard_normal((b, s, hkv, d)).astype(np.float32)).to(TORCH_DT[dtype]).cuda()
    print(f"varlen equal lengths vs batched {dtype} D{d} causal={causal}", flush=True)
    ob, lb = A.flash_attention(q, k, v, causal=causal, return_lse=True)
    cu = torch.arange(0, (b + 1) * s, s, dtype=torch.int32, device="cuda")
    ov, lv = A.varlen_attention(q.reshape(b * s, hq, d), k.reshape(b * s, hkv, d), v.reshape(b * s, hkv, d), cu, s,
                                causal=causal, return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(ov.reshape(b, s, hq, d), ob)
    assert torch.equal(lv.reshape(hq, b, s).permute(1, 0, 2), lb)


@pytest.mark.slow
def test_varlen_batched_short_sequences_full():
    """16 packed sequences, lengths uniform in [128, 512] (seeded), 32 heads,
    D = 64, fp16, non-causal: every output row against the oracle."""
    from transformer_attention_06_amd import workloads as W

    w = W.WORKLOADS["batched_varlen"]
    q, k, v, cu = W.make_varlen_inputs(w)
    qd, qn = prep(q, w.dtype)
    kd, kn = prep(k, w.dtype)
    vd, vn = prep(v, w.dtype)
    print(f"varlen full {w.name} T={q.shape[0]}", flush=True)
    o, l = _run((qd, kd, vd), cu, int(np.diff(cu).max()), w.causal)
    ro, rl = oracle.attention_varlen(qn, kn, vn, cu, causal=w.causal)
    assert_parity(o, ro, w.dtype, lse=l, lse_ref=rl, what=w.name)
