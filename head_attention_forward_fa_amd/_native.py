"""ctypes view of libmha_fwd.so (include/mha_fwd.h).  Argument marshalling
only: every step of the computation runs in the library's HIP kernels.

Loading fails loudly when the library has not been built; there is no
fallback implementation.
"""

from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmha_fwd.so")

MHA_DTYPE_F32 = 0
MHA_DTYPE_BF16 = 1
MHA_DTYPE_FP8_E4M3 = 2
MHA_DTYPE_FP8_E4M3_FASTACC = 3

MHA_OK = 0
MHA_ERR_INVALID_ARG = 1
MHA_ERR_UNSUPPORTED = 2
MHA_ERR_HIP = 3

EXPORTS = ("mha_fwd", "mha_fwd_last_error", "mha_fwd_supported", "mha_fwd_kernel_info",
           "mha_fwd_set_kernel_events", "mha_sched_visit", "mha_quantize_fp8",
           "mha_fwd_splitkv", "mha_combine_splits", "mha_fwd_auto_splits", "mha_fwd_noalloc")

_lib = None


class MhaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"mha status {status}: {msg}")
        self.status = status


def load() -> ctypes.CDLL:
    """Load (once) and type the library's exports."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with "
            "`python -m head_attention_forward_fa_amd.build` (hipcc, gfx950)")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float
    lib.mha_fwd.argtypes = [vp, vp, vp, vp, vp,        # q k v o lse
                            vp, i32, i32,              # cu_seqlens batch max_seqlen
                            i32, i32,                  # num_heads num_kv_heads
                            i32, i32, i32,             # Dn Dr Dv
                            vp, vp,                    # q_rope k_rope
                            i32, f32, i32,             # causal softmax_scale dtype
                            vp, vp, vp]                # q_scale k_scale stream
    lib.mha_fwd.restype = ctypes.c_int
    lib.mha_fwd_noalloc.argtypes = lib.mha_fwd.argtypes
    lib.mha_fwd_noalloc.restype = ctypes.c_int
    lib.mha_fwd_last_error.argtypes = []
    lib.mha_fwd_last_error.restype = ctypes.c_char_p
    lib.mha_fwd_supported.argtypes = [i32, i32, i32, i32]
    lib.mha_fwd_supported.restype = ctypes.c_int
    ip = ctypes.POINTER(ctypes.c_int32)
    lib.mha_fwd_kernel_info.argtypes = [i32, i32, i32, i32, ip, ip, ip, ip]
    lib.mha_fwd_kernel_info.restype = ctypes.c_int
    lib.mha_fwd_set_kernel_events.argtypes = [vp, vp]
    lib.mha_fwd_set_kernel_events.restype = ctypes.c_int
    lib.mha_sched_visit.argtypes = [vp, i32, i32, i32, i32, i32, i32, i32, i32, vp, vp]
    lib.mha_sched_visit.restype = ctypes.c_int
    lib.mha_quantize_fp8.argtypes = [vp, i32, ctypes.c_int64, i32, vp, vp, vp]
    lib.mha_quantize_fp8.restype = ctypes.c_int
    lib.mha_fwd_splitkv.argtypes = [vp, vp, vp, vp, vp,       # q k v o lse
                                    vp, i32, i32,             # cu_seqlens batch max_seqlen
                                    i32, i32,                 # num_heads num_kv_heads
                                    i32, i32, i32,            # Dn Dr Dv
                                    vp, vp,                   # q_rope k_rope
                                    i32, f32, i32,            # causal softmax_scale dtype
                                    vp, vp,                   # q_scale k_scale
                                    i32, i32, vp, vp, vp]     # T num_splits o_part lse_part stream
    lib.mha_fwd_splitkv.restype = ctypes.c_int
    lib.mha_combine_splits.argtypes = [vp, vp, i32, i32, i32, i32, i32, vp, vp, vp]
    lib.mha_combine_splits.restype = ctypes.c_int
    lib.mha_fwd_auto_splits.argtypes = [i32, i32, i32, i32, i32, i32]
    lib.mha_fwd_auto_splits.restype = ctypes.c_int
    _lib = lib
    return lib


def check(status: int) -> None:
    if status != MHA_OK:
        msg = load().mha_fwd_last_error().decode(errors="replace")
        if status in (MHA_ERR_INVALID_ARG, MHA_ERR_UNSUPPORTED):
            raise ValueError(f"mha status {status}: {msg}")
        raise MhaError(status, msg)
