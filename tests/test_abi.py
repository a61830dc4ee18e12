"""C-ABI checks that need no GPU: the library loads, exports every function
that include/*.h declares, and rejects bad arguments on the host (no HIP call
is made on any path exercised here)."""

import ctypes
import glob
import os
import re
import subprocess

import pytest

from transformer_attention_06_amd import attn as A

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        src = open(h).read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        for m in re.finditer(r"^[A-Za-z_][\w\s\*]*?\b(attn_\w+)\s*\(", src, flags=re.M):
            names.add(m.group(1))
    return sorted(names)


@pytest.fixture(scope="module")
def lib():
    return A.load_library()


def test_header_declares_entry_points():
    assert declared_functions() == sorted(A.EXPORTED_SYMBOLS)


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", A.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if l.strip()}
    for name in declared_functions():
        assert name in exported, name
        assert getattr(lib, name) is not None


def test_version_and_strerror(lib):
    assert A.version().startswith("attn_fwd ")
    assert "gfx950" in A.version()
    for code in range(-12, 1):
        assert A.strerror(code)
    assert A.strerror(-1234) == "unknown error code"


def test_library_built_from_the_tree(lib):
    """attn_version() names the sources the library was built from; the
    library under test must come from the sources in this tree."""
    from transformer_attention_06_amd.build import source_hash
    assert re.fullmatch(r"[0-9a-f]{16}", A.library_source_hash())
    assert A.library_source_hash() == source_hash()


FAKE = 0x10000  # a 16-byte aligned non-NULL address that is never dereferenced


def T(B=1, S=8, H=2, D=64, dtype=A.ATTN_BF16, data=FAKE):
    return A.AttnTensor(ctypes.c_void_p(data), dtype, B, S, H, D)


def call(lib, q, k, v, out, mask_kind=0, pad=None, scale=0.0, causal=0, hq=None, hkv=None, lse=None):
    hq = q.H if hq is None else hq
    hkv = k.H if hkv is None else hkv
    return lib.attn_fwd(ctypes.byref(q) if q is not None else None,
                        ctypes.byref(k) if k is not None else None,
                        ctypes.byref(v) if v is not None else None,
                        mask_kind, pad, ctypes.c_float(scale), causal, hq, hkv,
                        ctypes.byref(out) if out is not None else None, lse, None)


def test_null_descriptors(lib):
    assert call(lib, None, T(), T(), T(), hq=2, hkv=2) == A.ATTN_ERR_NULL
    assert call(lib, T(), T(), T(), None, hq=2, hkv=2) == A.ATTN_ERR_NULL


def test_null_data_pointer(lib):
    assert call(lib, T(data=0), T(), T(), T()) == A.ATTN_ERR_NULL


@pytest.mark.parametrize("field,val", [("B", 2), ("S", 9), ("D", 128)])
def test_shape_mismatch(lib, field, val):
    k = T()
    setattr(k, field, val)
    assert call(lib, T(), k, T(), T()) in (A.ATTN_ERR_SHAPE,)


def test_negative_dims(lib):
    assert call(lib, T(S=-1), T(S=-1), T(S=-1), T(S=-1)) == A.ATTN_ERR_SHAPE


def test_head_checks(lib):
    assert call(lib, T(H=4), T(H=3), T(H=3), T(H=4)) == A.ATTN_ERR_HEADS      # 4 % 3
    assert call(lib, T(H=4), T(H=2), T(H=2), T(H=4), hq=8) == A.ATTN_ERR_HEADS
    assert call(lib, T(H=4), T(H=2), T(H=1), T(H=4)) == A.ATTN_ERR_HEADS      # k.H != v.H
    assert call(lib, T(H=4), T(H=2), T(H=2), T(H=2), hq=4) == A.ATTN_ERR_HEADS  # out.H
    assert call(lib, T(H=2), T(H=2), T(H=2), T(H=2), hq=0, hkv=0) == A.ATTN_ERR_HEADS


def test_dtype_checks(lib):
    assert call(lib, T(dtype=7), T(), T(), T()) == A.ATTN_ERR_DTYPE
    assert call(lib, T(), T(dtype=A.ATTN_F16), T(), T()) == A.ATTN_ERR_DTYPE
    assert call(lib, T(), T(), T(), T(dtype=A.ATTN_F32)) == A.ATTN_ERR_DTYPE


@pytest.mark.parametrize("d", [1, 8, 24, 72, 264, 272, 512])
def test_unsupported_head_dim(lib, d):
    assert call(lib, T(D=d), T(D=d), T(D=d), T(D=d)) == A.ATTN_ERR_UNSUPPORTED


@pytest.mark.parametrize("d", [16, 32, 80, 96, 256])
def test_general_head_dim_16_bit_only(lib, d):
    # accepted for fp16/bf16 (the general kernel); fp32 keeps D in {64, 128}
    f32 = dict(dtype=A.ATTN_F32)
    assert call(lib, T(D=d, **f32), T(D=d, **f32), T(D=d, **f32), T(D=d, **f32)) == A.ATTN_ERR_UNSUPPORTED
    # a bf16 call with D = d passes every check (caught here on the null data pointer instead of a launch)
    assert call(lib, T(D=d, data=0), T(D=d), T(D=d), T(D=d)) == A.ATTN_ERR_NULL


def test_mask_checks(lib):
    assert call(lib, T(), T(), T(), T(), mask_kind=2) == A.ATTN_ERR_MASK
    assert call(lib, T(), T(), T(), T(), mask_kind=A.ATTN_MASK_KEY_PADDING, pad=None) == A.ATTN_ERR_MASK
    assert call(lib, T(), T(), T(), T(), mask_kind=A.ATTN_MASK_NONE, pad=FAKE) == A.ATTN_ERR_MASK
    assert call(lib, T(), T(), T(), T(), causal=2) == A.ATTN_ERR_MASK
    assert call(lib, T(), T(), T(), T(), mask_kind=A.ATTN_MASK_KEY_PADDING, pad=FAKE + 2) == A.ATTN_ERR_ALIGN


def test_alignment(lib):
    assert call(lib, T(data=FAKE + 8), T(), T(), T()) == A.ATTN_ERR_ALIGN
    assert call(lib, T(), T(), T(), T(data=FAKE + 2)) == A.ATTN_ERR_ALIGN
    assert call(lib, T(), T(), T(), T(), lse=FAKE + 1) == A.ATTN_ERR_ALIGN


def test_empty_inputs_return_ok_without_launch(lib):
    # B == 0 or S == 0: nothing to do, and no HIP call (this container has no GPU)
    assert call(lib, T(B=0), T(B=0), T(B=0), T(B=0)) == A.ATTN_OK
    assert call(lib, T(S=0), T(S=0), T(S=0), T(S=0)) == A.ATTN_OK
    assert call(lib, T(S=0, data=0), T(S=0, data=0), T(S=0, data=0), T(S=0, data=0)) == A.ATTN_OK


def test_size_limits(lib):
    big = dict(S=1 << 29)
    assert call(lib, T(**big), T(**big), T(**big), T(**big)) == A.ATTN_ERR_UNSUPPORTED
    assert call(lib, T(H=70000), T(H=1), T(H=1), T(H=70000)) == A.ATTN_ERR_UNSUPPORTED


def test_python_binding_rejects_cpu_tensors():
    import torch
    q = torch.zeros(1, 4, 1, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        A.attn_fwd(q, q, q, 0, None, None, False, 1, 1, q.clone(), None)


def test_missing_library_fails_loudly(tmp_path):
    import importlib
    saved = A._LIB
    try:
        A._LIB = None
        with pytest.raises(RuntimeError, match="missing"):
            A.load_library(str(tmp_path / "nope.so"))
    finally:
        A._LIB = saved


# --------------------------------------------------------------------------
# attn_fwd_rope: the same checks plus its own (k_rot, positions), host only
# --------------------------------------------------------------------------
def call_rope(lib, q, k, v, out, k_rot, positions=None, base=0.0, lse=None, causal=0):
    return lib.attn_fwd_rope(ctypes.byref(q), ctypes.byref(k), ctypes.byref(v), 0, None, ctypes.c_float(0.0),
                             causal, q.H, k.H, positions, ctypes.c_float(base),
                             ctypes.byref(k_rot) if k_rot is not None else None, ctypes.byref(out), lse, None)


# four disjoint fake buffers (bf16, 1x8x2x64 = 2 KiB each)
QA, KA, VA, OA, RA = (FAKE + i * 0x10000 for i in range(5))


def test_rope_shares_attention_checks(lib):
    assert call_rope(lib, T(H=4, data=QA), T(H=3, data=KA), T(H=3, data=VA), T(H=4, data=OA),
                     T(H=3, data=RA)) == A.ATTN_ERR_HEADS
    assert call_rope(lib, T(D=96, data=QA), T(D=96, data=KA), T(D=96, data=VA), T(D=96, data=OA),
                     T(D=96, data=RA)) == A.ATTN_ERR_UNSUPPORTED


def test_rope_k_rot_checks(lib):
    args = (T(data=QA), T(data=KA), T(data=VA), T(data=OA))
    assert call_rope(lib, *args, None) == A.ATTN_ERR_NULL
    assert call_rope(lib, *args, T(data=0)) == A.ATTN_ERR_NULL
    assert call_rope(lib, *args, T(data=RA, dtype=A.ATTN_F16)) == A.ATTN_ERR_DTYPE
    assert call_rope(lib, *args, T(data=RA, S=9)) == A.ATTN_ERR_SHAPE
    assert call_rope(lib, *args, T(data=RA, H=3)) == A.ATTN_ERR_SHAPE
    assert call_rope(lib, *args, T(data=RA + 8)) == A.ATTN_ERR_ALIGN
    assert call_rope(lib, *args, T(data=RA), positions=FAKE + 2) == A.ATTN_ERR_ALIGN


def test_rope_aliasing(lib):
    args = (T(data=QA), T(data=KA), T(data=VA), T(data=OA))
    nbytes = 1 * 8 * 2 * 64 * 2
    assert call_rope(lib, *args, T(data=QA)) == A.ATTN_ERR_ALIAS            # k_rot is q
    assert call_rope(lib, *args, T(data=VA + 16)) == A.ATTN_ERR_ALIAS       # overlaps v
    assert call_rope(lib, *args, T(data=OA - nbytes + 16)) == A.ATTN_ERR_ALIAS  # tail overlaps out
    assert call_rope(lib, *args, T(data=KA + 16)) == A.ATTN_ERR_ALIAS       # part of k
    assert call_rope(lib, *args, T(data=RA), lse=RA + 64) == A.ATTN_ERR_ALIAS


def test_rope_empty_inputs_return_ok_without_launch(lib):
    z = dict(S=0)
    assert call_rope(lib, T(**z), T(**z), T(**z), T(**z), T(**z)) == A.ATTN_OK
    z = dict(B=0, data=0)
    assert call_rope(lib, T(**z), T(**z), T(**z), T(**z), T(**z)) == A.ATTN_OK


# --------------------------------------------------------------------------
# attn_fwd_decode / attn_decode_workspace_bytes, host only
# --------------------------------------------------------------------------
def call_dec(lib, q, k, v, out, lens=None, causal=1, ws=FAKE + 0x100000, ws_bytes=1 << 30, lse=None):
    return lib.attn_fwd_decode(ctypes.byref(q), ctypes.byref(k), ctypes.byref(v), lens, ctypes.c_float(0.0),
                               causal, q.H, k.H, ctypes.byref(out), lse, ws, ctypes.c_int64(ws_bytes), None)


def test_decode_workspace_bytes(lib):
    # 1 KiB of arrival counters, then 256-key chunks x rows x (D + 3) floats
    c = A.DECODE_COUNTER_BYTES
    assert c == 1024
    assert A.decode_workspace_bytes(2, 1, 64, 128, 4096) == c + 16 * 2 * 64 * 1 * 131 * 4
    assert A.decode_workspace_bytes(1, 3, 8, 64, 1) == c + 1 * 1 * 8 * 3 * 67 * 4
    assert A.decode_workspace_bytes(1, 3, 8, 64, 257) == c + 2 * 1 * 8 * 3 * 67 * 4
    assert A.decode_workspace_bytes(1, 3, 8, 64, 0) == c + 1 * 1 * 8 * 3 * 67 * 4  # empty cache: one chunk
    assert lib.attn_decode_workspace_bytes(-1, 1, 1, 64, 1) == -1


def test_decode_checks(lib):
    q, k, v, o = T(S=1, H=8), T(S=100, H=2), T(S=100, H=2), T(S=1, H=8)
    assert call_dec(lib, q, k, T(S=99, H=2), o) == A.ATTN_ERR_SHAPE          # v length != k length
    assert call_dec(lib, q, k, v, T(S=2, H=8)) == A.ATTN_ERR_SHAPE           # out rows != q rows
    assert call_dec(lib, q, T(S=100, H=3), T(S=100, H=3), o) == A.ATTN_ERR_HEADS
    assert call_dec(lib, q, k, v, o, causal=3) == A.ATTN_ERR_MASK
    assert call_dec(lib, q, T(S=100, H=2, dtype=A.ATTN_F16), v, o) == A.ATTN_ERR_DTYPE
    assert call_dec(lib, T(S=1, H=8, D=96), T(S=100, H=2, D=96), T(S=100, H=2, D=96),
                    T(S=1, H=8, D=96)) == A.ATTN_ERR_UNSUPPORTED
    assert call_dec(lib, q, k, v, o, lens=FAKE + 2) == A.ATTN_ERR_ALIGN
    assert call_dec(lib, q, k, v, o, ws=None) == A.ATTN_ERR_NULL
    need = A.decode_workspace_bytes(1, 1, 8, 64, 100)
    assert call_dec(lib, q, k, v, o, ws_bytes=need - 1) == A.ATTN_ERR_WORKSPACE
    assert call_dec(lib, q, k, v, o, ws=FAKE + 0x100008) == A.ATTN_ERR_ALIGN


def test_decode_empty_queries_return_ok_without_launch(lib):
    assert call_dec(lib, T(S=0, H=8), T(S=100, H=2), T(S=100, H=2), T(S=0, H=8)) == A.ATTN_OK
    assert call_dec(lib, T(B=0, S=1, H=8, data=0), T(B=0, S=5, H=2, data=0), T(B=0, S=5, H=2, data=0),
                    T(B=0, S=1, H=8, data=0)) == A.ATTN_OK


# --------------------------------------------------------------------------
# attn_fwd_decode_noalloc: the same checks, and the fixed-workspace limit,
# all rejected before any HIP call
# --------------------------------------------------------------------------
def call_dec_na(lib, q, k, v, out, lens=None, causal=1, lse=None):
    return lib.attn_fwd_decode_noalloc(ctypes.byref(q), ctypes.byref(k), ctypes.byref(v), lens,
                                       ctypes.c_float(0.0), causal, q.H, k.H, ctypes.byref(out), lse, None)


def test_decode_noalloc_checks(lib):
    q, k, v, o = T(S=1, H=8), T(S=100, H=2), T(S=100, H=2), T(S=1, H=8)
    assert call_dec_na(lib, q, k, T(S=99, H=2), o) == A.ATTN_ERR_SHAPE
    assert call_dec_na(lib, q, T(S=100, H=3), T(S=100, H=3), o) == A.ATTN_ERR_HEADS
    assert call_dec_na(lib, q, k, v, o, causal=3) == A.ATTN_ERR_MASK
    assert call_dec_na(lib, q, k, v, o, lens=FAKE + 2) == A.ATTN_ERR_ALIGN
    assert call_dec_na(lib, T(S=1, H=8, data=0), k, v, o) == A.ATTN_ERR_NULL
    assert call_dec_na(lib, T(S=0, H=8), k, v, T(S=0, H=8)) == A.ATTN_OK  # no row: nothing launched


def test_decode_noalloc_rejects_sizes_beyond_its_workspace(lib):
    limit = 32 << 20
    # B=8, Hq=64, D=128, Sk=4096: 1 KiB + 16 chunks x 512 rows x 131 floats = 4.3 MB, within the limit
    assert A.decode_workspace_bytes(8, 1, 64, 128, 4096) <= limit
    # 16 times the cache: 68.7 MB, beyond it
    big = dict(B=8, H=8, D=128)
    assert A.decode_workspace_bytes(8, 1, 64, 128, 65536) > limit
    rc = call_dec_na(lib, T(S=1, B=8, H=64, D=128), T(S=65536, **big), T(S=65536, **big), T(S=1, B=8, H=64, D=128))
    assert rc == A.ATTN_ERR_SCRATCH
    assert "32 MiB" in A.strerror(rc)


# --------------------------------------------------------------------------
# attn_fwd_varlen: packed (1, T, H, D) buffers with offsets, host only
# --------------------------------------------------------------------------
def call_var(lib, q, k, v, out, cu=FAKE + 0x200000, n=3, max_len=8, causal=0, lse=None):
    return lib.attn_fwd_varlen(ctypes.byref(q), ctypes.byref(k), ctypes.byref(v), cu, n, ctypes.c_int64(max_len),
                               ctypes.c_float(0.0), causal, q.H, k.H, ctypes.byref(out), lse, None)


def test_varlen_checks(lib):
    q, k, v, o = T(S=20, H=4), T(S=20, H=2), T(S=20, H=2), T(S=20, H=4)
    assert call_var(lib, T(B=2, S=20, H=4), T(B=2, S=20, H=2), T(B=2, S=20, H=2),
                    T(B=2, S=20, H=4)) == A.ATTN_ERR_SHAPE                  # packed buffers have B == 1
    assert call_var(lib, q, k, T(S=19, H=2), o) == A.ATTN_ERR_SHAPE         # v rows != T
    assert call_var(lib, q, k, v, o, max_len=21) == A.ATTN_ERR_SHAPE         # longer than T
    assert call_var(lib, q, k, v, o, max_len=-1) == A.ATTN_ERR_SHAPE
    assert call_var(lib, q, k, v, o, n=-1) == A.ATTN_ERR_SHAPE
    assert call_var(lib, q, k, v, o, cu=None) == A.ATTN_ERR_NULL
    assert call_var(lib, q, k, v, o, cu=FAKE + 2) == A.ATTN_ERR_ALIGN
    assert call_var(lib, q, T(S=20, H=3), T(S=20, H=3), o) == A.ATTN_ERR_HEADS
    assert call_var(lib, q, k, v, o, causal=2) == A.ATTN_ERR_MASK
    assert call_var(lib, T(S=20, H=4, D=96), T(S=20, H=2, D=96), T(S=20, H=2, D=96),
                    T(S=20, H=4, D=96)) == A.ATTN_ERR_UNSUPPORTED
    assert call_var(lib, q, k, v, o, lse=FAKE + 2) == A.ATTN_ERR_ALIGN


def test_varlen_empty_returns_ok_without_launch(lib):
    q, k, v, o = T(S=20, H=4), T(S=20, H=2), T(S=20, H=2), T(S=20, H=4)
    assert call_var(lib, q, k, v, o, n=0) == A.ATTN_OK
    assert call_var(lib, q, k, v, o, max_len=0) == A.ATTN_OK
    z = dict(S=0, data=0)
    assert call_var(lib, T(H=4, **z), T(H=2, **z), T(H=2, **z), T(H=4, **z), max_len=0) == A.ATTN_OK


# --------------------------------------------------------------------------
# attn_fwd_masked: additive mask tensor, host only
# --------------------------------------------------------------------------
def call_mask(lib, q, k, v, out, mask=FAKE + 0x300000, mb=1, mh=1, causal=0, lse=None, mtype=0):
    return lib.attn_fwd_masked(ctypes.byref(q), ctypes.byref(k), ctypes.byref(v), mask, mtype, ctypes.c_int64(mb),
                               ctypes.c_int64(mh), ctypes.c_float(0.0), causal, q.H, k.H, ctypes.byref(out), lse,
                               None)


def test_masked_checks(lib):
    q, k, v, o = T(B=2, H=4), T(B=2, H=2), T(B=2, H=2), T(B=2, H=4)
    f32 = dict(dtype=A.ATTN_F32)
    assert call_mask(lib, T(B=2, H=4, **f32), T(B=2, H=2, **f32), T(B=2, H=2, **f32),
                     T(B=2, H=4, **f32)) == A.ATTN_ERR_UNSUPPORTED            # 16-bit types only
    assert call_mask(lib, q, k, v, o, mb=3) == A.ATTN_ERR_MASK                # batch dim neither 1 nor B
    assert call_mask(lib, q, k, v, o, mtype=2) == A.ATTN_ERR_MASK             # unknown mask type
    assert call_mask(lib, q, k, v, o, mtype=A.ATTN_MASK_BOOL, mask=FAKE + 8) == A.ATTN_ERR_ALIGN
    assert call_mask(lib, q, k, v, o, mh=2) == A.ATTN_ERR_MASK                # head dim neither 1 nor Hq
    assert call_mask(lib, q, k, v, o, mask=None) == A.ATTN_ERR_NULL
    assert call_mask(lib, q, k, v, o, mask=FAKE + 8) == A.ATTN_ERR_ALIGN
    assert call_mask(lib, q, k, v, o, causal=2) == A.ATTN_ERR_MASK
    assert call_mask(lib, q, T(B=2, H=3), T(B=2, H=3), o) == A.ATTN_ERR_HEADS
    assert call_mask(lib, T(B=2, H=4, D=72), T(B=2, H=2, D=72), T(B=2, H=2, D=72),
                     T(B=2, H=4, D=72)) == A.ATTN_ERR_UNSUPPORTED              # not a multiple of 16
    assert call_mask(lib, T(B=2, H=4, D=272), T(B=2, H=2, D=272), T(B=2, H=2, D=272),
                     T(B=2, H=4, D=272)) == A.ATTN_ERR_UNSUPPORTED             # above 256


def test_masked_empty_returns_ok_without_launch(lib):
    z = dict(S=0)
    assert call_mask(lib, T(H=4, **z), T(H=2, **z), T(H=2, **z), T(H=4, **z), mask=None) == A.ATTN_OK
