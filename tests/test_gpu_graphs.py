"""The newer entry points captured in a HIP graph: attn_fwd_decode (two
launches through a caller workspace), attn_fwd_varlen and attn_fwd_masked.
Each captured call is replayed several times, with eager work and
synchronisations in between and the outputs poisoned before every replay;
every replay must reproduce the eager result bit for bit."""

import numpy as np
import pytest
import torch

from gpu_helpers import prep
from transformer_attention_06_amd import attn as A

pytestmark = pytest.mark.gpu


def _replays(call, outs, ref, noise):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for i in range(4):
        for t in outs:
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for t, r in zip(outs, ref):
            assert torch.equal(t, r), f"replay {i}"
        noise()  # eager work between replays


def _t(rng, shape, dtype="bf16"):
    return prep(rng.standard_normal(shape).astype(np.float32), dtype)[0]


def test_graph_decode():
    rng = np.random.default_rng(41)
    B, Sq, Sk, Hq, Hkv, D = 2, 1, 1500, 16, 2, 128
    q, k, v = _t(rng, (B, Sq, Hq, D)), _t(rng, (B, Sk, Hkv, D)), _t(rng, (B, Sk, Hkv, D))
    lens = torch.tensor([1500, 700], dtype=torch.int32, device="cuda")
    ref_o, ref_l = A.decode_attention(q, k, v, cache_lens=lens, return_lse=True)
    out = torch.empty_like(q)
    lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device="cuda")
    ws = torch.zeros(A.decode_workspace_bytes(B, Sq, Hq, D, Sk), dtype=torch.uint8, device="cuda")
    print("graph case decode", flush=True)
    _replays(lambda: A.attn_fwd_decode(q, k, v, lens, None, True, Hq, Hkv, out, lse, ws), [out, lse],
             [ref_o, ref_l], lambda: A.decode_attention(q, k, v, causal=False))


def test_graph_varlen():
    rng = np.random.default_rng(42)
    lens = [130, 0, 257, 64]
    T, Hq, Hkv, D = sum(lens), 4, 2, 64
    q, k, v = _t(rng, (T, Hq, D), "fp16"), _t(rng, (T, Hkv, D), "fp16"), _t(rng, (T, Hkv, D), "fp16")
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]).astype(np.int32), device="cuda")
    ref_o, ref_l = A.varlen_attention(q, k, v, cu, max(lens), causal=True, return_lse=True)
    out = torch.zeros_like(q)
    lse = torch.full((Hq, T), float("-inf"), dtype=torch.float32, device="cuda")
    print("graph case varlen", flush=True)
    _replays(lambda: A.attn_fwd_varlen(q, k, v, cu, max(lens), None, True, Hq, Hkv, out, lse), [out, lse],
             [ref_o, ref_l], lambda: A.varlen_attention(q, k, v, cu, max(lens)))


def test_graph_masked():
    rng = np.random.default_rng(43)
    B, S, Hq, Hkv, D = 2, 300, 4, 2, 128
    q, k, v = _t(rng, (B, S, Hq, D)), _t(rng, (B, S, Hkv, D)), _t(rng, (B, S, Hkv, D))
    m = (rng.standard_normal((B, 1, S, S)) * 2).astype(np.float32)
    m[rng.random(m.shape) < 0.2] = -np.inf
    md = prep(m, "bf16")[0]
    ref_o, ref_l = A.masked_attention(q, k, v, md, causal=True, return_lse=True)
    out = torch.empty_like(q)
    lse = torch.empty((B, Hq, S), dtype=torch.float32, device="cuda")
    print("graph case masked", flush=True)
    _replays(lambda: A.attn_fwd_masked(q, k, v, md, None, True, Hq, Hkv, out, lse), [out, lse],
             [ref_o, ref_l], lambda: A.masked_attention(q, k, v, md))
