"""Seeded synthetic attention workloads.

This module only draws inputs: it holds none of the attention arithmetic, so
that both the HIP path and the fp64 oracle can be fed from it without sharing
any code.  Values are drawn as float32 with numpy's PCG64 generator, Q then K
then V (then any extras), each (B, S, H, D); the caller rounds them to the
storage dtype (round-to-nearest-even) before either side sees them.

The shapes stand in for the attention layers of the models the pages run
(Llama-2-7B with 32 heads of D=128, a Llama-2-70B-style GQA layer with 8 kv
heads, batched short sequences with D=64): no weights or datasets are used.
The fixed-pattern stress tensors (all zeros, all one large value, a heavy
tail) follow "ops-transformer：Transformer算子融合与推理加速实战" §4.2, which
warns that random inputs alone miss softmax saturation.
"""

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

MASK_NONE = 0
MASK_KEY_PADDING = 1


@dataclass(frozen=True)
class Workload:
    name: str
    index: int
    B: int
    S: int
    Hq: int
    Hkv: int
    D: int
    dtype: str                 # "fp32" | "fp16" | "bf16"
    causal: bool
    mask_kind: int = MASK_NONE
    pad_range: Optional[tuple] = None   # inclusive [lo, hi] for key padding
    outlier_frac: float = 0.0           # Bernoulli fraction scaled by outlier_mult
    outlier_mult: float = 1.0
    outlier_tensors: tuple = ("q", "k", "v")
    want_lse: bool = False
    note: str = ""
    extra: dict = field(default_factory=dict)

    @property
    def seed(self):
        return 42 + self.index


WORKLOADS = {
    "tiny_fp32": Workload(
        "tiny_fp32", 0, B=1, S=128, Hq=2, Hkv=2, D=64, dtype="fp32",
        causal=False, want_lse=True,
        note="oracle-check size; plus zeros / all-8.0 / Student-t(2) stress"),
    "llama2_7b_prefill": Workload(
        "llama2_7b_prefill", 1, B=1, S=2048, Hq=32, Hkv=32, D=128, dtype="bf16",
        causal=True, note="Llama-2-7B-shaped causal prefill"),
    "batched_padded": Workload(
        "batched_padded", 2, B=16, S=512, Hq=32, Hkv=32, D=64, dtype="fp16",
        causal=False, mask_kind=MASK_KEY_PADDING, pad_range=(128, 512),
        note="batched short sequences, per-sequence valid key lengths"),
    "batched_varlen": Workload(
        "batched_varlen", 2, B=16, S=512, Hq=32, Hkv=32, D=64, dtype="fp16",
        causal=False, pad_range=(128, 512),
        note="the batched short sequences packed back to back (no padding): "
             "16 lengths uniform in [128, 512]"),
    "gqa_llama2_70b": Workload(
        "gqa_llama2_70b", 3, B=2, S=4096, Hq=64, Hkv=8, D=128, dtype="bf16",
        causal=True, outlier_frac=0.01, outlier_mult=20.0,
        note="GQA 8:1, 1% of Q/K/V entries scaled by 20"),
    "gqa_llama2_70b_qk": Workload(
        "gqa_llama2_70b_qk", 3, B=2, S=4096, Hq=64, Hkv=8, D=128, dtype="bf16",
        causal=True, outlier_frac=0.01, outlier_mult=20.0,
        outlier_tensors=("q", "k"),
        note="as gqa_llama2_70b with outliers on Q and K only"),
    "long_context": Workload(
        "long_context", 4, B=1, S=16384, Hq=32, Hkv=32, D=128, dtype="bf16",
        causal=True, want_lse=True, note="long-context causal prefill, LSE on"),
}


def _draw(rng, shape, outlier_frac, outlier_mult, with_outliers):
    x = rng.standard_normal(shape, dtype=np.float32)
    if with_outliers and outlier_frac > 0.0:
        m = rng.random(shape) < outlier_frac
        x[m] *= np.float32(outlier_mult)
    return x


def make_inputs(w, seed=None, *, B=None, S=None):
    """Draw float32 Q, K, V (B,S,H,D) and int32 pad_lens (or None).

    ``B``/``S`` override the workload's sizes (reduced-size parity cases use
    the same distributions and structure).
    """
    rng = np.random.default_rng(w.seed if seed is None else seed)
    b = w.B if B is None else B
    s = w.S if S is None else S
    q = _draw(rng, (b, s, w.Hq, w.D), w.outlier_frac, w.outlier_mult, "q" in w.outlier_tensors)
    k = _draw(rng, (b, s, w.Hkv, w.D), w.outlier_frac, w.outlier_mult, "k" in w.outlier_tensors)
    v = _draw(rng, (b, s, w.Hkv, w.D), w.outlier_frac, w.outlier_mult, "v" in w.outlier_tensors)
    pad = None
    if w.mask_kind == MASK_KEY_PADDING:
        lo, hi = w.pad_range
        lo, hi = min(lo, s), min(hi, s)
        pad = rng.integers(lo, hi, size=b, endpoint=True).astype(np.int32)
    return q, k, v, pad


def make_varlen_inputs(w, seed=None):
    """Packed sequences: draw the B lengths (uniform in w.pad_range), then
    float32 Q (T, Hq, D), K and V (T, Hkv, D) for T = the sum of the lengths.
    Returns q, k, v and the int64 offsets cu[0..B] (cu[0] = 0)."""
    rng = np.random.default_rng(w.seed if seed is None else seed)
    lo, hi = w.pad_range
    lens = rng.integers(lo, hi, size=w.B, endpoint=True)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    t = int(cu[-1])
    q = rng.standard_normal((t, w.Hq, w.D), dtype=np.float32)
    k = rng.standard_normal((t, w.Hkv, w.D), dtype=np.float32)
    v = rng.standard_normal((t, w.Hkv, w.D), dtype=np.float32)
    return q, k, v, cu


def random_inputs(seed, B, S, Hq, Hkv, D, *, dist="normal", df=2.0):
    """Generic seeded draw for parity sweeps: Q, K, V float32 (B,S,H,D)."""
    rng = np.random.default_rng(seed)
    if dist == "normal":
        f = lambda shp: rng.standard_normal(shp, dtype=np.float32)
    elif dist == "student_t":
        f = lambda shp: rng.standard_t(df, size=shp).astype(np.float32)
    elif dist == "uniform":
        f = lambda shp: rng.uniform(-1.0, 1.0, size=shp).astype(np.float32)
    else:
        raise ValueError(dist)
    return f((B, S, Hq, D)), f((B, S, Hkv, D)), f((B, S, Hkv, D))


def random_pad_lens(seed, B, lo, hi):
    rng = np.random.default_rng(seed)
    return rng.integers(lo, hi, size=B, endpoint=True).astype(np.int32)


def stress_inputs(kind, B=1, S=128, H=2, D=64, seed=42):
    """Fixed-pattern stress tensors: 'zeros', 'const8' (all 8.0) or
    'student_t' (iid Student-t with 2 degrees of freedom)."""
    shape = (B, S, H, D)
    if kind == "zeros":
        z = np.zeros(shape, np.float32)
        return z, z.copy(), z.copy()
    if kind == "const8":
        c = np.full(shape, 8.0, np.float32)
        return c, c.copy(), c.copy()
    if kind == "student_t":
        rng = np.random.default_rng(seed)
        return tuple(rng.standard_t(2.0, size=shape).astype(np.float32) for _ in range(3))
    raise ValueError(kind)
