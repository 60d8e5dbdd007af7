"""Fused multi-head-attention forward pass for AMD Instinct MI355X (gfx950).

The computation lives in libmha_fwd.so (HIP kernels behind the C ABI of
include/mha_fwd.h); this package is its thin PyTorch binding.
"""

from .mha import (  # noqa: F401
    mha_combine_splits, mha_fwd, mha_fwd_auto_splits, mha_fwd_kernel_info, mha_fwd_noalloc,
    mha_fwd_supported, mha_quantize_fp8, mha_sched_visit,
)
from ._native import (  # noqa: F401
    MHA_DTYPE_BF16, MHA_DTYPE_F32, MHA_DTYPE_FP8_E4M3, MHA_DTYPE_FP8_E4M3_FASTACC, MhaError, load,
)
