"""CPU oracle for the fused multi-head-attention forward pass.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library and
its Python binding) may import, call or execute anything in this package.  It
is used by ``tests/``, by ``__graft_entry__.smoke()`` and by the
``cpu_baseline`` leg of ``bench.py``, and by nothing else.

It evaluates the plain definition of attention directly in float64 (numpy),
with the full score matrix and an ordinary softmax: no tiling, no online
softmax, no reordering.  It shares no code with the HIP path.
"""

from .attention import (  # noqa: F401
    decode_bf16,
    decode_e4m3,
    dequantize_per_token,
    default_softmax_scale,
    mha_forward,
    mha_forward_rows,
)
