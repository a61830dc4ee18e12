"""ATTN_LOG=1: every launch names its kernel variant, grid and workgroup size
on stderr (checked in a child process, where the variable is read once)."""

import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = """
import torch
from transformer_attention_06_amd import attn as A
q = torch.randn(1, 256, 2, 128, device="cuda").to(torch.bfloat16)
k = torch.randn(1, 256, 2, 128, device="cuda").to(torch.bfloat16)
v = torch.randn(1, 256, 2, 128, device="cuda").to(torch.bfloat16)
out = torch.empty_like(q)
A.attn_fwd(q, k, v, A.ATTN_MASK_NONE, None, None, True, 2, 2, out, None)
m = torch.zeros(1, 1, 256, 256, device="cuda").to(torch.bfloat16)
A.masked_attention(q, k, v, m, causal=True)
qs, ks, vs = (x[:, :200].contiguous() for x in (q, k, v))
A.masked_attention(qs, ks, vs, torch.ones(1, 1, 200, 200, dtype=torch.bool, device="cuda"), causal=True)
torch.cuda.synchronize()
print("done", flush=True)
"""


def _run(env_value):
    env = dict(os.environ)
    if env_value is None:
        env.pop("ATTN_LOG", None)
    else:
        env["ATTN_LOG"] = env_value
    return subprocess.run([sys.executable, "-c", CHILD], cwd=ROOT, env=env, capture_output=True, text=True,
                          timeout=300)


def test_attn_log_names_the_variant():
    r = _run("1")
    assert r.returncode == 0, r.stderr[-3000:]
    assert "done" in r.stdout
    assert "[attn] attn_fwd_kernel<bf16, D=128, causal=1, pad=0, lse=0, rope=0, mask=0> groups=2 grid=2 block=512" \
        in r.stderr
    # a mask tensor with rows of 16-byte multiples takes the tuned kernel,
    # a boolean one with S % 16 != 0 the general kernel
    assert "[attn] attn_fwd_kernel<bf16, D=128, causal=1, pad=0, lse=0, rope=0, mask=1> groups=2 grid=2" in r.stderr
    assert "[attn] masked_kernel<bf16, DP=128, causal=1, mask_mode=3" in r.stderr


def test_no_log_without_the_variable():
    r = _run("0")
    assert r.returncode == 0, r.stderr[-3000:]
    assert "[attn]" not in r.stderr
