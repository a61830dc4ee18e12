"""The error emulator (tests/emulator.py), pinned on the CPU.

In fp64 with no rounding (exact=True) its tile-by-tile recurrence must equal
the plain oracle to rounding, for every mask combination and ragged lengths;
its bfloat16 rounding must agree with torch's (an independent library
conversion); and with the kernel's roundings its error stays inside the
parity bars on inputs shaped like the benchmark workloads."""

import numpy as np
import pytest
import torch

import oracle
from emulator import emulate_head, round_bf16
from tolerances import BAR


@pytest.mark.parametrize("S,D,causal,key_len", [(1, 8, False, None), (50, 16, True, None), (64, 32, False, 37),
                                                 (129, 64, True, 100), (200, 16, True, 0), (257, 8, False, 256)])
def test_exact_recurrence_equals_oracle(S, D, causal, key_len):
    rng = np.random.default_rng(S + D)
    q, k, v = (rng.standard_normal((S, D)) * 3 for _ in range(3))
    scale = 1.0 / np.sqrt(D)
    ro, rl = oracle.attention_head(q, k, v, scale, causal=causal, key_len=key_len)
    eo, el = emulate_head(q, k, v, scale, "bf16", causal=causal, key_len=key_len, exact=True)
    np.testing.assert_allclose(eo, ro, rtol=0, atol=1e-12)
    fin = np.isfinite(rl)
    assert np.array_equal(fin, np.isfinite(el))
    np.testing.assert_allclose(el[fin], rl[fin], rtol=0, atol=1e-12)


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(5)
    x = np.concatenate([rng.standard_normal(100000) * 10.0 ** rng.integers(-8, 8, 100000),
                        np.array([0.0, -0.0, 1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -9, 65504.0])]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(round_bf16(x).view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("dtype,causal", [("bf16", True), ("fp16", False)])
def test_rounded_error_inside_bars(dtype, causal):
    S, D = 256, 128
    rng = np.random.default_rng(9)
    q, k, v = (rng.standard_normal((S, D)).astype(np.float32) for _ in range(3))
    q, k, v = (torch.from_numpy(x).to(torch.bfloat16 if dtype == "bf16" else torch.float16).float().numpy()
               .astype(np.float64) for x in (q, k, v))
    scale = 1.0 / np.sqrt(D)
    ro, rl = oracle.attention_head(q, k, v, scale, causal=causal)
    eo, el = emulate_head(q, k, v, scale, dtype, causal=causal)
    err = np.abs(eo - ro)
    assert 0 < err.max() <= BAR[dtype]["max_abs"] and err.mean() <= BAR[dtype]["mean_abs"]
    assert np.abs(el - rl).max() <= 1e-3
