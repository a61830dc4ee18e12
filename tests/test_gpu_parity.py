"""HIP path vs the fp64 oracle, element by element, through the C ABI.

Small sizes span several 128-row query blocks and 64-key tiles with ragged
tails; the five workload shapes run in the same launch configuration the
benchmark times, checked in full where the oracle finishes in seconds and on
sampled rows (plus size-independent properties) where it does not.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import prep, run, to_np
from tolerances import assert_parity, fp32_sensitivity_bound, lse_error
from transformer_attention_06_amd import attn as A
from transformer_attention_06_amd import workloads as W

pytestmark = pytest.mark.gpu


def _oracle(qn, kn, vn, causal, pad, scale=None):
    mk = oracle.MASK_NONE if pad is None else oracle.MASK_KEY_PADDING
    return oracle.attention(qn, kn, vn, causal=causal, mask_kind=mk, pad_lens=pad, scale=scale)


def _case(seed, B, S, Hq, Hkv, D, dtype, causal, padded, dist="normal"):
    q, k, v = W.random_inputs(seed, B, S, Hq, Hkv, D, dist=dist)
    pad = W.random_pad_lens(seed + 1, B, 0, S) if padded else None
    qd, qn = prep(q, dtype)
    kd, kn = prep(k, dtype)
    vd, vn = prep(v, dtype)
    out, lse = run(qd, kd, vd, causal=causal, pad=pad)
    ro, rl = _oracle(qn, kn, vn, causal, pad)
    return to_np(out), to_np(lse), ro, rl


# --------------------------------------------------------------------------
# tile-edge sweep: every dtype, head dim, mask combination and GQA grouping
# --------------------------------------------------------------------------
SWEEP_S = [1, 2, 31, 64, 65, 128, 129, 200, 300]


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("padded", [False, True])
def test_sweep(dtype, D, causal, padded):
    for n, S in enumerate(SWEEP_S):
        for (Hq, Hkv) in ((2, 2), (6, 2)):
            seed = 1000 + 17 * n + Hq
            o, l, ro, rl = _case(seed, 2, S, Hq, Hkv, D, dtype, causal, padded)
            assert_parity(o, ro, dtype, lse=l, lse_ref=rl,
                          what=f"{dtype} D{D} S{S} H{Hq}/{Hkv} c{causal} p{padded}")


def test_gqa_group_sizes():
    for (Hq, Hkv) in ((8, 1), (8, 4), (16, 2), (3, 1)):
        o, l, ro, rl = _case(7, 1, 160, Hq, Hkv, 128, "bf16", True, False)
        assert_parity(o, ro, "bf16", lse=l, lse_ref=rl, what=f"gqa {Hq}/{Hkv}")


# --------------------------------------------------------------------------
# tiny fp32 workload and its fixed-pattern stress tensors
# --------------------------------------------------------------------------
def test_tiny_fp32_normal():
    w = W.WORKLOADS["tiny_fp32"]
    q, k, v, _ = W.make_inputs(w)
    qd, qn = prep(q, "fp32")
    kd, kn = prep(k, "fp32")
    vd, vn = prep(v, "fp32")
    out, lse = run(qd, kd, vd)
    ro, rl = _oracle(qn, kn, vn, False, None)
    e = assert_parity(to_np(out), ro, "fp32", lse=to_np(lse), lse_ref=rl, what="tiny fp32")
    assert e["max_abs"] <= 1e-5


@pytest.mark.parametrize("kind", ["zeros", "const8"])
def test_tiny_fp32_stress_closed_forms(kind):
    q, k, v = W.stress_inputs(kind)
    qd, _ = prep(q, "fp32")
    kd, _ = prep(k, "fp32")
    vd, _ = prep(v, "fp32")
    out, lse = run(qd, kd, vd)
    fill = 0.0 if kind == "zeros" else 8.0
    o = to_np(out)
    assert np.all(o == fill)
    exp_lse = fill * fill * 64 / 8 + math.log(128.0)
    assert np.abs(to_np(lse) - exp_lse).max() <= 1e-3


def test_tiny_fp32_student_t():
    q, k, v = W.stress_inputs("student_t")
    qd, qn = prep(q, "fp32")
    kd, kn = prep(k, "fp32")
    vd, vn = prep(v, "fp32")
    out, lse = run(qd, kd, vd)
    ro, rl = _oracle(qn, kn, vn, False, None)
    bound = fp32_sensitivity_bound(qn, kn, vn, 1.0 / 8.0)
    err = np.abs(to_np(out) - ro)
    assert np.all(err <= bound), f"max ratio {np.max(err / bound)}"
    assert lse_error(to_np(lse), rl) <= 1e-3


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_stress_16bit(dtype):
    for kind in ("zeros", "const8"):
        q, k, v = W.stress_inputs(kind, S=200, D=128)
        qd, _ = prep(q, dtype)
        kd, _ = prep(k, dtype)
        vd, _ = prep(v, dtype)
        out, lse = run(qd, kd, vd, causal=True)
        fill = 0.0 if kind == "zeros" else 8.0
        assert np.all(to_np(out) == fill), kind
        exp_lse = fill * fill * 128 / math.sqrt(128) + np.log(np.arange(1, 201))
        assert np.abs(to_np(lse)[0] - exp_lse[None, :]).max() <= 1e-3


# --------------------------------------------------------------------------
# closed forms on the GPU
# --------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
def test_uniform_scores_prefix_mean(dtype):
    """Q = 0: O_i = mean of V[0..i] under causal masking, LSE_i = ln(i+1)."""
    S, D = 300, 64
    rng = np.random.default_rng(5)
    v = rng.standard_normal((1, S, 1, D)).astype(np.float32)
    k = rng.standard_normal((1, S, 1, D)).astype(np.float32)
    qd, _ = prep(np.zeros((1, S, 1, D), np.float32), dtype)
    kd, _ = prep(k, dtype)
    vd, vn = prep(v, dtype)
    out, lse = run(qd, kd, vd, causal=True)
    ref = np.cumsum(vn[0, :, 0, :].astype(np.float64), axis=0) / np.arange(1, S + 1)[:, None]
    assert_parity(to_np(out)[0, :, 0, :], ref, dtype, what="prefix mean")
    assert np.abs(to_np(lse)[0, 0] - np.log(np.arange(1, S + 1))).max() <= 1e-3


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_one_hot_selection(dtype):
    """Q_i = 480·e_{pi(i)}, K_j = e_j (scale 1/8): score margin 60, O_i = V[pi(i)]."""
    S, D = 64, 64
    perm = np.roll(np.arange(S), 5) % D
    q = np.zeros((1, S, 1, D), np.float32)
    k = np.zeros((1, S, 1, D), np.float32)
    for i in range(S):
        q[0, i, 0, perm[i]] = 480.0
        k[0, i, 0, i] = 1.0
    v = np.random.default_rng(3).standard_normal((1, S, 1, D)).astype(np.float32)
    qd, _ = prep(q, dtype)
    kd, _ = prep(k, dtype)
    vd, vn = prep(v, dtype)
    out, lse = run(qd, kd, vd)
    o = to_np(out)[0, :, 0, :]
    assert_parity(o, vn[0, perm, 0, :], dtype, what="one-hot")
    assert np.abs(to_np(lse)[0, 0] - 60.0).max() <= 1e-3


def test_first_causal_row_and_single_key():
    for S in (1, 77):
        o, l, ro, rl = _case(11, 2, S, 4, 2, 128, "bf16", True, False)
        q, k, v = W.random_inputs(11, 2, S, 4, 2, 128)
        vb = torch.from_numpy(v).to(torch.bfloat16).float().numpy()
        for b in range(2):
            for h in range(4):
                assert np.array_equal(o[b, 0, h], vb[b, 0, h // 2])
        assert_parity(o, ro, "bf16", lse=l, lse_ref=rl, what=f"S={S}")


def test_fully_masked_batch_rows():
    """pad_lens = 0 for a batch: O = 0 and LSE = -inf, never NaN."""
    q, k, v = W.random_inputs(3, 3, 100, 2, 2, 64)
    qd, qn = prep(q, "bf16")
    kd, kn = prep(k, "bf16")
    vd, vn = prep(v, "bf16")
    pad = np.array([0, 100, 37], np.int32)
    for causal in (False, True):
        out, lse = run(qd, kd, vd, causal=causal, pad=pad)
        o, l = to_np(out), to_np(lse)
        assert np.all(o[0] == 0.0) and np.all(np.isneginf(l[0]))
        ro, rl = _oracle(qn, kn, vn, causal, pad)
        assert_parity(o, ro, "bf16", lse=l, lse_ref=rl, what="masked batch")


def test_pad_lens_clamped():
    """Lengths outside [0, S] are clamped on the device."""
    q, k, v = W.random_inputs(4, 2, 90, 2, 2, 64)
    qd, qn = prep(q, "fp16")
    kd, kn = prep(k, "fp16")
    vd, vn = prep(v, "fp16")
    out, lse = run(qd, kd, vd, pad=np.array([-5, 1000], np.int32))
    ro, rl = _oracle(qn, kn, vn, False, np.array([0, 90], np.int32))
    assert_parity(to_np(out), ro, "fp16", lse=to_np(lse), lse_ref=rl, what="clamp")


def test_scale_default_and_explicit():
    q, k, v = W.random_inputs(9, 1, 150, 2, 2, 128)
    qd, qn = prep(q, "bf16")
    kd, kn = prep(k, "bf16")
    vd, vn = prep(v, "bf16")
    o1, l1 = run(qd, kd, vd, scale=None)
    o2, l2 = run(qd, kd, vd, scale=1.0 / math.sqrt(128))
    o3, l3 = run(qd, kd, vd, scale=-1.0)
    assert torch.equal(o1, o2) and torch.equal(o1, o3) and torch.equal(l1, l2)
    o4, l4 = run(qd, kd, vd, scale=0.05)
    ro, rl = _oracle(qn, kn, vn, False, None, scale=0.05)
    assert_parity(to_np(o4), ro, "bf16", lse=to_np(l4), lse_ref=rl, what="scale 0.05")


# --------------------------------------------------------------------------
# kernel-level properties
# --------------------------------------------------------------------------
def test_gqa_equals_expanded_mha():
    q, k, v = W.random_inputs(21, 2, 257, 8, 2, 128)
    qd, _ = prep(q, "bf16")
    kd, _ = prep(k, "bf16")
    vd, _ = prep(v, "bf16")
    o1, l1 = run(qd, kd, vd, causal=True)
    ke = kd.repeat_interleave(4, dim=2).contiguous()
    ve = vd.repeat_interleave(4, dim=2).contiguous()
    o2, l2 = run(qd, ke, ve, causal=True)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_deterministic():
    q, k, v = W.random_inputs(22, 1, 700, 4, 4, 128)
    qd, _ = prep(q, "bf16")
    kd, _ = prep(k, "bf16")
    vd, _ = prep(v, "bf16")
    o1, l1 = run(qd, kd, vd, causal=True)
    o2, l2 = run(qd, kd, vd, causal=True)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_output_guard_regions_untouched():
    """Writes stay inside out and lse: NaN guards around both are intact."""
    B, S, H, D = 2, 129, 2, 64
    q, k, v = W.random_inputs(23, B, S, H, H, D)
    qd, _ = prep(q, "fp16")
    kd, _ = prep(k, "fp16")
    vd, _ = prep(v, "fp16")
    n = B * S * H * D
    guard = 4096
    buf = torch.full((n + 2 * guard,), float("nan"), dtype=torch.float16, device="cuda")
    out = buf[guard:guard + n].view(B, S, H, D)
    lbuf = torch.full((B * H * S + 2 * guard,), float("nan"), dtype=torch.float32, device="cuda")
    lse = lbuf[guard:guard + B * H * S].view(B, H, S)
    A.attn_fwd(qd, kd, vd, A.ATTN_MASK_NONE, None, None, True, H, H, out, lse)
    torch.cuda.synchronize()
    assert torch.isnan(buf[:guard]).all() and torch.isnan(buf[guard + n:]).all()
    assert torch.isnan(lbuf[:guard]).all() and torch.isnan(lbuf[guard + B * H * S:]).all()
    assert not torch.isnan(out).any() and not torch.isnan(lse).any()


def test_no_device_allocation_per_call():
    q, k, v = W.random_inputs(24, 1, 256, 4, 4, 128)
    qd, _ = prep(q, "bf16")
    kd, _ = prep(k, "bf16")
    vd, _ = prep(v, "bf16")
    out = torch.empty_like(qd)
    lse = torch.empty((1, 4, 256), dtype=torch.float32, device="cuda")
    A.attn_fwd(qd, kd, vd, 0, None, None, True, 4, 4, out, lse)
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated()
    for _ in range(200):
        A.attn_fwd(qd, kd, vd, 0, None, None, True, 4, 4, out, lse)
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() == before


def test_empty_inputs_on_device():
    for shape in ((0, 16, 2, 64), (2, 0, 2, 64)):
        x = torch.empty(shape, dtype=torch.bfloat16, device="cuda")
        o = torch.empty_like(x)
        A.attn_fwd(x, x, x, 0, None, None, True, 2, 2, o, None)


def test_noncontiguous_rejected():
    x = torch.zeros(1, 64, 2, 128, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        A.flash_attention(x.transpose(1, 2), x.transpose(1, 2), x.transpose(1, 2))


def test_graph_replay_matches_eager():
    """A captured launch replayed several times, with eager work and
    synchronisations in between, reproduces the eager result every time."""
    q, k, v = W.random_inputs(25, 1, 333, 4, 2, 128)
    qd, _ = prep(q, "bf16")
    kd, _ = prep(k, "bf16")
    vd, _ = prep(v, "bf16")
    ref_o, ref_l = run(qd, kd, vd, causal=True)
    out = torch.empty_like(qd)
    lse = torch.empty((1, 4, 333), dtype=torch.float32, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        A.attn_fwd(qd, kd, vd, 0, None, None, True, 4, 2, out, lse)
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        A.attn_fwd(qd, kd, vd, 0, None, None, True, 4, 2, out, lse)
    for i in range(4):
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_o) and torch.equal(lse, ref_l), f"replay {i}"
        run(qd, kd, vd, causal=False)  # eager work between replays


# --------------------------------------------------------------------------
# work order: a multiple of 8 (batch, query head) units, so each XCD's range
# of units is used; without causal masking a unit's query blocks run one
# after another, under causal masking the pairs split the heavy block at
# its last tiles, and an odd block count leaves an unpaired middle block
# --------------------------------------------------------------------------
@pytest.mark.parametrize("dtype,D,causal,padded", [
    ("fp16", 64, False, True),    # three wavefronts per SIMD, task-minor order
    ("bf16", 64, False, False),
    ("bf16", 128, False, True),
    ("bf16", 128, True, False),   # causal pairs, middle block alone
    ("fp16", 64, True, True),
    ("fp32", 64, False, False),
])
def test_work_order_shapes(dtype, D, causal, padded):
    for (S, Hq, Hkv) in ((640, 8, 2), (384, 4, 4), (1152, 8, 8)):
        print(f"work order case {dtype} D{D} S{S} H{Hq}/{Hkv} causal={causal} padded={padded}", flush=True)
        o, l, ro, rl = _case(4242 + S + Hq, 2, S, Hq, Hkv, D, dtype, causal, padded)
        assert_parity(o, ro, dtype, lse=l, lse_ref=rl,
                      what=f"work order {dtype} D{D} S{S} H{Hq}/{Hkv} c{causal} p{padded}")
