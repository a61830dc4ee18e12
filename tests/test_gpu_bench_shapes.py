"""Parity at the full sizes and launch configurations bench.py times for its
extra lines (--masked, --general-d, --decode), on sampled heads or sequences
the fp64 oracle computes in seconds: every output row of those heads is
compared, in the same call that produced the whole tensor."""

import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import prep, to_np
from tolerances import assert_parity
from transformer_attention_06_amd import attn as A
from transformer_attention_06_amd import workloads as W

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

HEADS = [0, 13, 31]


def _llama_inputs(D, seed):
    w = W.Workload(f"llama2_7b_prefill_d{D}", 1, B=1, S=2048, Hq=32, Hkv=32, D=D, dtype="bf16", causal=True)
    q, k, v, _ = W.make_inputs(w, seed=seed)
    return prep(q, "bf16"), prep(k, "bf16"), prep(v, "bf16")


def test_masked_bench_shape():
    """bench.py --masked: B1 H32 S2048 D128 bf16, causal flag plus a (1, 1, S, S)
    mask of N(0,1)·0.5 shifts with -inf above the diagonal."""
    (qd, qn), (kd, kn), (vd, vn) = _llama_inputs(128, 43)
    S = 2048
    rng = np.random.default_rng(143)
    m = (rng.standard_normal((1, 1, S, S)) * 0.5).astype(np.float32)
    m[0, 0][np.triu(np.ones((S, S), bool), 1)] = -np.inf
    md, mn = prep(m, "bf16")
    print("bench-shape case masked", flush=True)
    out, lse = A.masked_attention(qd, kd, vd, md, causal=True, return_lse=True)
    torch.cuda.synchronize()
    o, l = to_np(out), lse.cpu().numpy()
    ro, rl = oracle.attention_masked(qn[:, :, HEADS], kn[:, :, HEADS], vn[:, :, HEADS], mn, causal=True)
    assert_parity(o[:, :, HEADS], ro, "bf16", lse=l[:, HEADS], lse_ref=rl, what="masked bench shape")


@pytest.mark.parametrize("D", [80, 96, 160, 256])
def test_general_d_bench_shape(D):
    """bench.py --general-d: B1 H32 S2048 bf16 causal at the general kernel's
    head dims."""
    (qd, qn), (kd, kn), (vd, vn) = _llama_inputs(D, 44 + D)
    print(f"bench-shape case general D{D}", flush=True)
    out, lse = A.flash_attention(qd, kd, vd, causal=True, return_lse=True)
    torch.cuda.synchronize()
    o, l = to_np(out), lse.cpu().numpy()
    ro, rl = oracle.attention(qn[:, :, HEADS], kn[:, :, HEADS], vn[:, :, HEADS], causal=True)
    assert_parity(o[:, :, HEADS], ro, "bf16", lse=l[:, HEADS], lse_ref=rl, what=f"general D{D} bench shape")


def test_decode_mha_bench_shape():
    """bench.py --decode, Llama-2-7B-shaped multi-head decode: B16 Sq1 Sk4096
    H32 D128 bf16; sequences 0, 7 and 15 against the oracle."""
    B, Sq, Sk, H, D = 16, 1, 4096, 32, 128
    rng = np.random.default_rng(45)
    q = rng.standard_normal((B, Sq, H, D)).astype(np.float32)
    k = rng.standard_normal((B, Sk, H, D)).astype(np.float32)
    v = rng.standard_normal((B, Sk, H, D)).astype(np.float32)
    (qd, qn), (kd, kn), (vd, vn) = prep(q, "bf16"), prep(k, "bf16"), prep(v, "bf16")
    print("bench-shape case MHA decode", flush=True)
    out, lse = A.decode_attention(qd, kd, vd, causal=True, return_lse=True)
    torch.cuda.synchronize()
    o, l = to_np(out), lse.cpu().numpy()
    bs = [0, 7, 15]
    ro, rl = oracle.attention_decode(qn[bs], kn[bs], vn[bs], causal=True)
    assert_parity(o[bs], ro, "bf16", lse=l[bs], lse_ref=rl, what="MHA decode bench shape")
