"""Shared plumbing for the GPU parity tests (inputs in, outputs back)."""

import numpy as np
import torch

from transformer_attention_06_amd import attn as A

TORCH_DT = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}


def prep(x, dtype):
    """float32 numpy -> (device tensor in dtype, float32 numpy of the rounded
    values the kernel reads; exact for bf16/fp16)."""
    t = torch.from_numpy(np.ascontiguousarray(x)).to(TORCH_DT[dtype])
    return t.cuda(), t.to(torch.float32).numpy()


def run(qd, kd, vd, *, causal=False, pad=None, scale=None, lse=True):
    pad_d = None if pad is None else torch.from_numpy(np.asarray(pad, np.int32)).cuda()
    out, l = A.flash_attention(qd, kd, vd, causal=causal, pad_lens=pad_d, scale=scale, return_lse=True)
    torch.cuda.synchronize()
    return out, l


def to_np(t):
    return t.to(torch.float32).cpu().numpy()
