"""Plain CPU oracle for per-token fp8 quantisation of Q or K rows.

TEST INFRASTRUCTURE ONLY: imported by tests/ and __graft_entry__.smoke(),
never by the product path.

The attention kernel takes Q and K as 8-bit floats with one float32 scale per
(token, head) row (SM100AttentionSMem, Parameters: scale_dtype_, the per-token
scale of Q and K; Methods q_scale_smem / k_scale_smem hold BM resp. BN of
them per tile).  The pages do not say how the codes and scales are made.
Reading used here (the one the fp8 inputs are generated with):

    scale = amax(|row|) / 448          (448: largest finite OCP E4M3 value;
                                        a row of zeros gets scale 1)
    code  = E4M3 value nearest to clamp(x / scale, -448, 448),
            ties to the code with an even mantissa (round to nearest even)

Precision: the division and the clamp are float32 operations, as on the
device, because they decide integer codes; everything else is exact.  The
rounding itself is done by searching the table of all finite E4M3 values
(from their bit-level definition in oracle.attention.decode_e4m3) for the
nearest one, so no floating-point conversion routine is involved.
"""

from __future__ import annotations

import numpy as np

from .attention import decode_bf16, decode_e4m3

E4M3_MAX = 448.0


def e4m3_table():
    """(values float64 [127], codes uint8 [127]) of the non-negative finite
    E4M3 codes 0x00 .. 0x7E, ascending in value."""
    codes = np.arange(0x7F, dtype=np.uint8)
    vals = decode_e4m3(codes)
    order = np.argsort(vals, kind="stable")
    return vals[order], codes[order]


def round_to_e4m3(y: np.ndarray) -> np.ndarray:
    """float32 values already inside [-448, 448] -> E4M3 codes (uint8).

    Magnitude: the nearest entry of the value table; at an exact midpoint the
    code whose mantissa (bit 0 of the code) is even.  Sign: bit 7 from the
    sign of y (so -0.0 gives 0x80).
    """
    y = np.asarray(y, dtype=np.float32)
    if np.any(np.abs(y) > E4M3_MAX) or np.any(np.isnan(y)):
        raise ValueError("round_to_e4m3 expects finite values within +-448")
    vals, codes = e4m3_table()
    a = np.abs(y.astype(np.float64)).ravel()
    hi = np.clip(np.searchsorted(vals, a, side="left"), 0, len(vals) - 1)
    lo = np.clip(hi - 1, 0, len(vals) - 1)
    d_lo = a - vals[lo]
    d_hi = vals[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & ((codes[hi] & 1) == 0))
    mag = np.where(pick_hi, codes[hi], codes[lo]).astype(np.uint8)
    sign = np.signbit(y.ravel()).astype(np.uint8) << np.uint8(7)
    return (mag | sign).reshape(y.shape)


def quantize_rows(x: np.ndarray):
    """Rows [..., D] (float32 values) -> (codes uint8 [..., D], scales float32 [...]).

    One scale per row of the last axis (a (token, head) row of a [T, H, D]
    tensor).
    """
    x = np.asarray(x, dtype=np.float32)
    amax = np.abs(x).max(axis=-1)
    scale = np.where(amax > 0, (amax / np.float32(E4M3_MAX)).astype(np.float32),
                     np.float32(1.0)).astype(np.float32)
    y = (x / scale[..., None]).astype(np.float32)
    y = np.clip(y, np.float32(-E4M3_MAX), np.float32(E4M3_MAX))
    return round_to_e4m3(y), scale


def quantize_bf16_rows(bits: np.ndarray):
    """bfloat16 bit patterns [..., D] -> (codes, scales) of quantize_rows."""
    return quantize_rows(decode_bf16(bits).astype(np.float32))
