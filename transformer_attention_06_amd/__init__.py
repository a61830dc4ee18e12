"""MI355X-native fused attention forward (gfx950 HIP kernels behind a C ABI).

``transformer_attention_06_amd.attn`` holds the ctypes binding of the C-ABI
library ``libattn_fwd.so``; ``workloads`` draws the seeded synthetic inputs.
Nothing is loaded at import time: the binding loads the library on first use
and raises if it has not been built.
"""

__all__ = ["attn", "workloads"]
