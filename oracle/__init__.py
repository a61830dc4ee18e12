"""CPU fp64 oracle for the fused attention forward.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute anything in this package: only the tests, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with
the HIP path (no kernels, headers, helpers, tables or pre/post-processing) and
imports nothing from the ``transformer_attention_06_amd`` package.

Pages cited (short name -> page title / address):

* [ops-transformer]  "ops-transformer：Transformer算子融合与推理加速实战"
  (xdnf.cn/news/343851)
* [graph-opt]        "CANN-ATB图优化-昇腾NPU怎么把PyTorch计算图改造成融合算子"
  (adg.csdn.net/6a3125fb10ee7a33f27dfef6)
* [ATB-guide]        the ATB engineering guide at
  hwcomputing.csdn.net/6a59a88310ee7a33f28e5ce9
* [ops+ATB]          "CANN-ops-transformer和ATB-昇腾NPU上算子和加速库怎么配合"
  (lpnh.cn/news/719634)

Parity status: every function here is pinned by the ``-m "not gpu"`` tests in
``tests/test_oracle_pins.py`` (closed forms, invariants, an independent
library routine and a high-precision brute force); none is "parity unpinned".
The rotary embedding (``rope``) is pinned the same way by
``tests/oracle_rope_pins.py`` (closed forms at D = 2, 4, 8, rotation
invariants, the relative-position property and the complex-number form), and
decode attention over a KV cache (``attention_decode``) by
``tests/oracle_decode_pins.py`` (equality with the last rows of a prefill,
cache truncation, the key-split merge by LSE, torch's SDPA), and attention over packed
variable-length sequences (``attention_varlen``) by
``tests/oracle_varlen_pins.py`` (the batched oracle at equal lengths, key
padding standing in for a shorter sequence, torch's SDPA per sequence, the
uniform-score closed form, independence of sequences), and attention under
an explicit additive mask tensor (``attention_masked``) by
``tests/oracle_masked_pins.py`` (the prefill oracle for zero, triangular and
key-padding masks, torch's SDPA with a float mask under every broadcast
shape, the per-row shift invariance, fully masked rows).
"""

from .attention import (  # noqa: F401
    MASK_NONE,
    MASK_KEY_PADDING,
    default_scale,
    kv_head_for,
    allowed_keys,
    attention_head,
    attention,
    attention_rows,
)
from .rope import (  # noqa: F401
    DEFAULT_BASE as ROPE_DEFAULT_BASE,
    rope_frequencies,
    rope_positions,
    rope,
)
from .decode import (  # noqa: F401
    visible_keys as decode_visible_keys,
    attention_decode,
)
from .varlen import (  # noqa: F401
    check_offsets as varlen_check_offsets,
    attention_varlen,
)
from .masked import (  # noqa: F401
    mask_slice,
    additive_from_bool,
    attention_masked,
)
