"""attn_fwd_decode_noalloc (decode with the library's fixed per-GPU workspace)
against attn_fwd_decode with a caller workspace: both run the same kernels, so
the outputs and LSE must be identical, bit for bit, on two calls in a row (the
second smaller, so it runs over what the first left in the array).  Neither
the binding nor the library allocates: torch's allocator reports no new
device memory across the call."""

import pytest
import torch

from transformer_attention_06_amd import attn as A

pytestmark = pytest.mark.gpu


def _inputs(seed, B, Sq, Sk, Hq, Hkv, D, dtype, lens):
    g = torch.Generator(device="cuda").manual_seed(seed)
    q = torch.randn(B, Sq, Hq, D, device="cuda", generator=g).to(dtype)
    k = torch.randn(B, Sk, Hkv, D, device="cuda", generator=g).to(dtype)
    v = torch.randn(B, Sk, Hkv, D, device="cuda", generator=g).to(dtype)
    cl = torch.tensor(lens, dtype=torch.int32, device="cuda")
    return q, k, v, cl


CASES = [
    # (seed, B, Sq, Sk, Hq, Hkv, D, dtype, cache lens, causal)
    (11, 4, 2, 1000, 16, 4, 128, torch.bfloat16, [1000, 517, 256, 3], True),
    (12, 2, 1, 300, 8, 8, 64, torch.float16, [300, 129], False),
]


def _run_pair(case):
    seed, B, Sq, Sk, Hq, Hkv, D, dtype, lens, causal = case
    q, k, v, cl = _inputs(seed, B, Sq, Sk, Hq, Hkv, D, dtype, lens)
    ref_o = torch.full_like(q, float("nan"))
    ref_l = torch.full((B, Hq, Sq), float("nan"), dtype=torch.float32, device="cuda")
    ws = torch.zeros(A.decode_workspace_bytes(B, Sq, Hq, D, Sk), dtype=torch.uint8, device="cuda")
    A.attn_fwd_decode(q, k, v, cl, None, causal, Hq, Hkv, ref_o, ref_l, ws)
    out = torch.full_like(q, float("nan"))
    lse = torch.full((B, Hq, Sq), float("nan"), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated()
    A.attn_fwd_decode_noalloc(q, k, v, cl, None, causal, Hq, Hkv, out, lse)
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() == before
    assert torch.isfinite(out.float()).all() and not torch.isnan(lse).any()
    assert torch.equal(out.view(torch.int16), ref_o.view(torch.int16)), f"outputs differ: {case[:8]}"
    assert torch.equal(lse, ref_l), f"LSE differs: {case[:8]}"


def test_noalloc_matches_workspace_entry_twice_second_smaller():
    for case in CASES:  # the second call is smaller than the first
        _run_pair(case)


def test_noalloc_rejects_oversize_without_launch():
    q = torch.zeros(8, 1, 64, 128, dtype=torch.bfloat16, device="cuda")
    k = torch.zeros(8, 65536, 8, 128, dtype=torch.bfloat16, device="cuda")
    out = torch.empty_like(q)
    with pytest.raises(A.AttnArgumentError) as e:
        A.attn_fwd_decode_noalloc(q, k, k, None, None, True, 64, 8, out, None)
    assert e.value.code == A.ATTN_ERR_SCRATCH
