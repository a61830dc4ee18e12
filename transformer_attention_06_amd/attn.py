"""Python binding of libattn_fwd.so (argument marshalling only).

Every step of the attention forward runs in the library's HIP kernels; this
module only turns torch tensors into the C descriptors of ``include/attn_fwd.h``
and passes torch's current HIP stream.  If the library has not been built,
loading it raises: there is no Python or CPU fallback.
"""

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libattn_fwd.so")

ATTN_F32, ATTN_F16, ATTN_BF16 = 0, 1, 2
ATTN_MASK_NONE, ATTN_MASK_KEY_PADDING = 0, 1

ATTN_OK = 0
ATTN_ERR_NULL = -1
ATTN_ERR_SHAPE = -2
ATTN_ERR_HEADS = -3
ATTN_ERR_DTYPE = -4
ATTN_ERR_UNSUPPORTED = -5
ATTN_ERR_MASK = -6
ATTN_ERR_ALIGN = -7
ATTN_ERR_LAUNCH = -8
ATTN_ERR_DEVICE = -9
ATTN_ERR_ALIAS = -10
ATTN_ERR_WORKSPACE = -11
ATTN_ERR_SCRATCH = -12
ATTN_MASK_ADDITIVE = 0
ATTN_MASK_BOOL = 1

EXPORTED_SYMBOLS = ("attn_fwd", "attn_fwd_varlen", "attn_fwd_masked", "attn_fwd_rope", "attn_fwd_decode",
                    "attn_fwd_decode_noalloc", "attn_decode_workspace_bytes", "attn_strerror", "attn_version")


class AttnTensor(ctypes.Structure):
    """Mirror of ``attn_tensor_t``: a contiguous (B, S, H, D) device buffer."""

    _fields_ = [
        ("data", ctypes.c_void_p),
        ("dtype", ctypes.c_int32),
        ("B", ctypes.c_int64),
        ("S", ctypes.c_int64),
        ("H", ctypes.c_int64),
        ("D", ctypes.c_int64),
    ]


_LIB = None


def load_library(path=LIB_PATH):
    """Load libattn_fwd.so once and declare its C signatures."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python -m transformer_attention_06_amd.build` "
            "(hipcc, gfx950). There is no fallback path.")
    lib = ctypes.CDLL(path)
    P = ctypes.POINTER(AttnTensor)
    lib.attn_fwd.argtypes = [P, P, P, ctypes.c_int, ctypes.c_void_p, ctypes.c_float, ctypes.c_int,
                             ctypes.c_int, ctypes.c_int, P, ctypes.c_void_p, ctypes.c_void_p]
    lib.attn_fwd.restype = ctypes.c_int
    lib.attn_fwd_varlen.argtypes = [P, P, P, ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float,
                                    ctypes.c_int, ctypes.c_int, ctypes.c_int, P, ctypes.c_void_p, ctypes.c_void_p]
    lib.attn_fwd_varlen.restype = ctypes.c_int
    lib.attn_fwd_masked.argtypes = [P, P, P, ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_int64, ctypes.c_float,
                                    ctypes.c_int, ctypes.c_int, ctypes.c_int, P, ctypes.c_void_p, ctypes.c_void_p]
    lib.attn_fwd_masked.restype = ctypes.c_int
    lib.attn_fwd_rope.argtypes = [P, P, P, ctypes.c_int, ctypes.c_void_p, ctypes.c_float, ctypes.c_int,
                                  ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_float, P, P,
                                  ctypes.c_void_p, ctypes.c_void_p]
    lib.attn_fwd_rope.restype = ctypes.c_int
    lib.attn_fwd_decode.argtypes = [P, P, P, ctypes.c_void_p, ctypes.c_float, ctypes.c_int, ctypes.c_int,
                                    ctypes.c_int, P, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                    ctypes.c_void_p]
    lib.attn_fwd_decode.restype = ctypes.c_int
    lib.attn_fwd_decode_noalloc.argtypes = [P, P, P, ctypes.c_void_p, ctypes.c_float, ctypes.c_int, ctypes.c_int,
                                            ctypes.c_int, P, ctypes.c_void_p, ctypes.c_void_p]
    lib.attn_fwd_decode_noalloc.restype = ctypes.c_int
    lib.attn_decode_workspace_bytes.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int, ctypes.c_int64,
                                                ctypes.c_int64]
    lib.attn_decode_workspace_bytes.restype = ctypes.c_int64
    lib.attn_strerror.argtypes = [ctypes.c_int]
    lib.attn_strerror.restype = ctypes.c_char_p
    lib.attn_version.argtypes = []
    lib.attn_version.restype = ctypes.c_char_p
    _LIB = lib
    return lib


def strerror(code):
    return load_library().attn_strerror(int(code)).decode()


def version():
    return load_library().attn_version().decode()


def library_source_hash():
    """Hash of the sources the loaded library was built from (the last word
    of attn_version())."""
    return version().rsplit(" ", 1)[-1]


class AttnError(RuntimeError):
    def __init__(self, code):
        self.code = code
        super().__init__(f"attn_fwd failed ({code}): {strerror(code)}")


class AttnArgumentError(AttnError, ValueError):
    pass


def check(code):
    if code == ATTN_OK:
        return
    if code in (ATTN_ERR_LAUNCH, ATTN_ERR_DEVICE):
        raise AttnError(code)
    raise AttnArgumentError(code)


def _dtype_code(t):
    import torch
    codes = {torch.float32: ATTN_F32, torch.float16: ATTN_F16, torch.bfloat16: ATTN_BF16}
    if t.dtype not in codes:
        raise AttnArgumentError(ATTN_ERR_DTYPE)
    return codes[t.dtype]


def describe(t):
    """AttnTensor for a contiguous 4-D (B, S, H, D) torch tensor."""
    if t.dim() != 4:
        raise AttnArgumentError(ATTN_ERR_SHAPE)
    if not t.is_contiguous():
        raise ValueError("attn_fwd needs contiguous (B, S, H, D) tensors")
    b, s, h, d = t.shape
    return AttnTensor(ctypes.c_void_p(t.data_ptr()), _dtype_code(t), b, s, h, d)


def _common_ptrs(q, k, v, out, pad_lens, lse, n_q_heads):
    import torch
    for name, t in (("q", q), ("k", k), ("v", v), ("out", out)):
        if not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
    pad_ptr = None
    if pad_lens is not None:
        if pad_lens.dtype != torch.int32 or not pad_lens.is_cuda or not pad_lens.is_contiguous():
            raise ValueError("pad_lens must be a contiguous int32 device tensor")
        pad_ptr = ctypes.c_void_p(pad_lens.data_ptr())
    lse_ptr = None
    if lse is not None:
        if lse.dtype != torch.float32 or not lse.is_cuda or not lse.is_contiguous():
            raise ValueError("lse must be a contiguous float32 device tensor")
        if tuple(lse.shape) != (q.shape[0], n_q_heads, q.shape[1]):
            raise ValueError("lse must be [B, n_q_heads, S]")
        lse_ptr = ctypes.c_void_p(lse.data_ptr())
    return pad_ptr, lse_ptr


def attn_fwd_rope(q, k, v, mask_kind, pad_lens, scale, causal, n_q_heads, n_kv_heads, positions,
                  rope_base, k_rot, out, lse, stream=None):
    """``attn_fwd_rope`` with torch tensors: RoPE(K) into ``k_rot``, then the
    attention of RoPE(Q), RoPE(K), V into ``out`` (and ``lse``).

    positions: int32 device tensor [B, S] or None (0 .. S-1); rope_base:
    float (None or <= 0 selects 10000); k_rot: tensor shaped like k (may be k).
    """
    import torch
    lib = load_library()
    pad_ptr, lse_ptr = _common_ptrs(q, k, v, out, pad_lens, lse, n_q_heads)
    if not k_rot.is_cuda:
        raise ValueError("k_rot must be a device tensor")
    pos_ptr = None
    if positions is not None:
        if positions.dtype != torch.int32 or not positions.is_cuda or not positions.is_contiguous():
            raise ValueError("positions must be a contiguous int32 device tensor")
        if tuple(positions.shape) != (q.shape[0], q.shape[1]):
            raise ValueError("positions must be [B, S]")
        pos_ptr = ctypes.c_void_p(positions.data_ptr())
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    dq, dk, dv, dkr, do = describe(q), describe(k), describe(v), describe(k_rot), describe(out)
    code = lib.attn_fwd_rope(ctypes.byref(dq), ctypes.byref(dk), ctypes.byref(dv), int(mask_kind), pad_ptr,
                             ctypes.c_float(0.0 if scale is None else float(scale)), int(bool(causal)),
                             int(n_q_heads), int(n_kv_heads), pos_ptr,
                             ctypes.c_float(0.0 if rope_base is None else float(rope_base)),
                             ctypes.byref(dkr), ctypes.byref(do), lse_ptr, ctypes.c_void_p(stream.cuda_stream))
    check(code)
    return out, k_rot, lse


def attn_fwd(q, k, v, mask_kind, pad_lens, scale, causal, n_q_heads, n_kv_heads, out, lse,
             stream=None):
    """The C entry point with torch tensors: fills ``out`` (and ``lse``).

    q, k, v, out: contiguous device tensors (B, S, H, D) of one dtype;
    pad_lens: int32 device tensor [B] or None; lse: float32 device tensor
    [B, n_q_heads, S] or None; scale: float (<= 0 or None selects 1/sqrt(D));
    stream: a torch stream (default: the current stream).
    """
    import torch
    lib = load_library()
    pad_ptr, lse_ptr = _common_ptrs(q, k, v, out, pad_lens, lse, n_q_heads)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    dq, dk, dv, do = describe(q), describe(k), describe(v), describe(out)
    code = lib.attn_fwd(ctypes.byref(dq), ctypes.byref(dk), ctypes.byref(dv), int(mask_kind), pad_ptr,
                        ctypes.c_float(0.0 if scale is None else float(scale)), int(bool(causal)),
                        int(n_q_heads), int(n_kv_heads), ctypes.byref(do), lse_ptr,
                        ctypes.c_void_p(stream.cuda_stream))
    check(code)
    return out, lse


def flash_attention(q, k, v, *, causal=False, pad_lens=None, scale=None, return_lse=False):
    """Allocate ``out`` (and ``lse``) with torch and run ``attn_fwd``.

    q: (B, S, Hq, D); k, v: (B, S, Hkv, D); pad_lens: int32 [B] or None.
    Returns out, or (out, lse) with lse float32 [B, Hq, S].
    """
    import torch
    out = torch.empty_like(q)
    lse = None
    if return_lse:
        lse = torch.empty((q.shape[0], q.shape[2], q.shape[1]), dtype=torch.float32, device=q.device)
    mask_kind = ATTN_MASK_NONE if pad_lens is None else ATTN_MASK_KEY_PADDING
    attn_fwd(q, k, v, mask_kind, pad_lens, scale, causal, q.shape[2], k.shape[2], out, lse)
    return (out, lse) if return_lse else out


def describe_packed(t):
    """AttnTensor (B = 1, S = T) for a contiguous 3-D (T, H, D) torch tensor."""
    if t.dim() != 3:
        raise AttnArgumentError(ATTN_ERR_SHAPE)
    return describe(t.unsqueeze(0))


def attn_fwd_varlen(q, k, v, cu_seqlens, max_seqlen, scale, causal, n_q_heads, n_kv_heads, out, lse,
                    stream=None):
    """``attn_fwd_varlen`` with torch tensors: packed sequences, sequence b
    at rows [cu_seqlens[b], cu_seqlens[b+1]) of q/out (T, Hq, D) and k/v
    (T, Hkv, D).  cu_seqlens: int32 device tensor [B+1]; max_seqlen: int
    bound on every length; lse: float32 device tensor [Hq, T] or None."""
    import torch
    lib = load_library()
    for name, t in (("q", q), ("k", k), ("v", v), ("out", out)):
        if not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
    if cu_seqlens.dtype != torch.int32 or not cu_seqlens.is_cuda or not cu_seqlens.is_contiguous() \
            or cu_seqlens.dim() != 1 or cu_seqlens.numel() < 1:
        raise ValueError("cu_seqlens must be a contiguous 1-D int32 device tensor of B+1 offsets")
    lse_ptr = None
    if lse is not None:
        if lse.dtype != torch.float32 or not lse.is_cuda or not lse.is_contiguous():
            raise ValueError("lse must be a contiguous float32 device tensor")
        if tuple(lse.shape) != (n_q_heads, q.shape[0]):
            raise ValueError("lse must be [n_q_heads, T]")
        lse_ptr = ctypes.c_void_p(lse.data_ptr())
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    dq, dk, dv, do = describe_packed(q), describe_packed(k), describe_packed(v), describe_packed(out)
    code = lib.attn_fwd_varlen(ctypes.byref(dq), ctypes.byref(dk), ctypes.byref(dv),
                               ctypes.c_void_p(cu_seqlens.data_ptr()), int(cu_seqlens.numel() - 1),
                               int(max_seqlen), ctypes.c_float(0.0 if scale is None else float(scale)),
                               int(bool(causal)), int(n_q_heads), int(n_kv_heads), ctypes.byref(do), lse_ptr,
                               ctypes.c_void_p(stream.cuda_stream))
    check(code)
    return out, lse


def varlen_attention(q, k, v, cu_seqlens, max_seqlen, *, causal=False, scale=None, return_lse=False):
    """Allocate ``out`` (zero-filled: rows outside every sequence stay 0) and
    ``lse`` with torch and run ``attn_fwd_varlen``.  Returns out, or
    (out, lse) with lse float32 [Hq, T]."""
    import torch
    out = torch.zeros_like(q)
    lse = None
    if return_lse:
        lse = torch.full((q.shape[1], q.shape[0]), float("-inf"), dtype=torch.float32, device=q.device)
    attn_fwd_varlen(q, k, v, cu_seqlens, max_seqlen, scale, causal, q.shape[1], k.shape[1], out, lse)
    return (out, lse) if return_lse else out


def attn_fwd_masked(q, k, v, mask, scale, causal, n_q_heads, n_kv_heads, out, lse, stream=None):
    """``attn_fwd_masked`` with torch tensors: q, k, v, out as for attn_fwd
    (bf16/fp16); mask: contiguous (1 or B, 1 or Hq, S, S) device tensor,
    either of q's dtype (added to the scaled scores, -inf hides a key) or
    torch.bool (True: the key takes part)."""
    import torch
    lib = load_library()
    _, lse_ptr = _common_ptrs(q, k, v, out, None, lse, n_q_heads)
    if not mask.is_cuda or not mask.is_contiguous() or mask.dim() != 4:
        raise ValueError("mask must be a contiguous 4-D device tensor (1|B, 1|Hq, S, S)")
    if mask.dtype == torch.bool:
        mask_type = ATTN_MASK_BOOL
    elif mask.dtype == q.dtype:
        mask_type = ATTN_MASK_ADDITIVE
    else:
        raise AttnArgumentError(ATTN_ERR_DTYPE)
    if tuple(mask.shape[2:]) != (q.shape[1], q.shape[1]):
        raise AttnArgumentError(ATTN_ERR_MASK)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    dq, dk, dv, do = describe(q), describe(k), describe(v), describe(out)
    code = lib.attn_fwd_masked(ctypes.byref(dq), ctypes.byref(dk), ctypes.byref(dv), ctypes.c_void_p(mask.data_ptr()),
                               int(mask_type), int(mask.shape[0]), int(mask.shape[1]),
                               ctypes.c_float(0.0 if scale is None else float(scale)), int(bool(causal)),
                               int(n_q_heads), int(n_kv_heads), ctypes.byref(do), lse_ptr,
                               ctypes.c_void_p(stream.cuda_stream))
    check(code)
    return out, lse


def masked_attention(q, k, v, mask, *, causal=False, scale=None, return_lse=False):
    """Allocate ``out`` (and ``lse``) with torch and run ``attn_fwd_masked``.
    Returns out, or (out, lse) with lse float32 [B, Hq, S]."""
    import torch
    out = torch.empty_like(q)
    lse = None
    if return_lse:
        lse = torch.empty((q.shape[0], q.shape[2], q.shape[1]), dtype=torch.float32, device=q.device)
    attn_fwd_masked(q, k, v, mask, scale, causal, q.shape[2], k.shape[2], out, lse)
    return (out, lse) if return_lse else out


def rope_attention(q, k, v, *, causal=False, pad_lens=None, scale=None, positions=None, rope_base=None,
                   return_lse=False):
    """Allocate ``out``, ``k_rot`` (and ``lse``) with torch and run
    ``attn_fwd_rope``.  Returns (out, k_rot) or (out, k_rot, lse)."""
    import torch
    out = torch.empty_like(q)
    k_rot = torch.empty_like(k)
    lse = None
    if return_lse:
        lse = torch.empty((q.shape[0], q.shape[2], q.shape[1]), dtype=torch.float32, device=q.device)
    mask_kind = ATTN_MASK_NONE if pad_lens is None else ATTN_MASK_KEY_PADDING
    attn_fwd_rope(q, k, v, mask_kind, pad_lens, scale, causal, q.shape[2], k.shape[2], positions, rope_base,
                  k_rot, out, lse)
    return (out, k_rot, lse) if return_lse else (out, k_rot)


# Leading bytes of every decode workspace that hold the arrival counters of
# the in-kernel split merge (zero between calls).
DECODE_COUNTER_BYTES = 1024


def decode_workspace_bytes(B, Sq, n_q_heads, D, Sk):
    """Bytes of workspace attn_fwd_decode needs (its first
    DECODE_COUNTER_BYTES must be zero before the first call; allocate it
    with torch.zeros and reuse it)."""
    return int(load_library().attn_decode_workspace_bytes(int(B), int(Sq), int(n_q_heads), int(D), int(Sk)))


def attn_fwd_decode(q, k_cache, v_cache, cache_lens, scale, causal, n_q_heads, n_kv_heads, out, lse,
                    workspace, stream=None):
    """``attn_fwd_decode`` with torch tensors: q/out (B, Sq, Hq, D), caches
    (B, Sk, Hkv, D), cache_lens int32 [B] or None, workspace a uint8 device
    tensor of at least decode_workspace_bytes(...) bytes whose first
    DECODE_COUNTER_BYTES are zero (every call leaves them zero)."""
    import torch
    lib = load_library()
    for name, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache), ("out", out), ("workspace", workspace)):
        if not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
    lens_ptr = None
    if cache_lens is not None:
        if cache_lens.dtype != torch.int32 or not cache_lens.is_cuda or not cache_lens.is_contiguous():
            raise ValueError("cache_lens must be a contiguous int32 device tensor")
        lens_ptr = ctypes.c_void_p(cache_lens.data_ptr())
    lse_ptr = None
    if lse is not None:
        if lse.dtype != torch.float32 or not lse.is_cuda or not lse.is_contiguous():
            raise ValueError("lse must be a contiguous float32 device tensor")
        if tuple(lse.shape) != (q.shape[0], n_q_heads, q.shape[1]):
            raise ValueError("lse must be [B, n_q_heads, Sq]")
        lse_ptr = ctypes.c_void_p(lse.data_ptr())
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    dq, dk, dv, do = describe(q), describe(k_cache), describe(v_cache), describe(out)
    code = lib.attn_fwd_decode(ctypes.byref(dq), ctypes.byref(dk), ctypes.byref(dv), lens_ptr,
                               ctypes.c_float(0.0 if scale is None else float(scale)), int(bool(causal)),
                               int(n_q_heads), int(n_kv_heads), ctypes.byref(do), lse_ptr,
                               ctypes.c_void_p(workspace.data_ptr()),
                               ctypes.c_int64(workspace.numel() * workspace.element_size()),
                               ctypes.c_void_p(stream.cuda_stream))
    check(code)
    return out, lse


def attn_fwd_decode_noalloc(q, k_cache, v_cache, cache_lens, scale, causal, n_q_heads, n_kv_heads, out, lse,
                            stream=None):
    """``attn_fwd_decode_noalloc`` with torch tensors (as attn_fwd_decode,
    without a workspace).  Marshals only: nothing is allocated here or in the
    library."""
    import torch
    lib = load_library()
    for name, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache), ("out", out)):
        if not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
    lens_ptr = None
    if cache_lens is not None:
        if cache_lens.dtype != torch.int32 or not cache_lens.is_cuda or not cache_lens.is_contiguous():
            raise ValueError("cache_lens must be a contiguous int32 device tensor")
        lens_ptr = ctypes.c_void_p(cache_lens.data_ptr())
    lse_ptr = None
    if lse is not None:
        if lse.dtype != torch.float32 or not lse.is_cuda or not lse.is_contiguous():
            raise ValueError("lse must be a contiguous float32 device tensor")
        if tuple(lse.shape) != (q.shape[0], n_q_heads, q.shape[1]):
            raise ValueError("lse must be [B, n_q_heads, Sq]")
        lse_ptr = ctypes.c_void_p(lse.data_ptr())
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    dq, dk, dv, do = describe(q), describe(k_cache), describe(v_cache), describe(out)
    code = lib.attn_fwd_decode_noalloc(ctypes.byref(dq), ctypes.byref(dk), ctypes.byref(dv), lens_ptr,
                                       ctypes.c_float(0.0 if scale is None else float(scale)), int(bool(causal)),
                                       int(n_q_heads), int(n_kv_heads), ctypes.byref(do), lse_ptr,
                                       ctypes.c_void_p(stream.cuda_stream))
    check(code)
    return out, lse


def decode_attention(q, k_cache, v_cache, *, cache_lens=None, causal=True, scale=None, return_lse=False):
    """Allocate ``out``, the workspace (and ``lse``) with torch and run
    ``attn_fwd_decode``.  Returns out, or (out, lse)."""
    import torch
    B, Sq, Hq, D = q.shape
    out = torch.empty_like(q)
    lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=q.device) if return_lse else None
    ws = torch.zeros(max(16, decode_workspace_bytes(B, Sq, Hq, D, k_cache.shape[1])), dtype=torch.uint8,
                     device=q.device)
    attn_fwd_decode(q, k_cache, v_cache, cache_lens, scale, causal, Hq, k_cache.shape[2], out, lse, ws)
    return (out, lse) if return_lse else out

