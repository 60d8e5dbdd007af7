"""Seeded synthetic inputs for the MHA forward pass.

This module only draws random numbers and stores them in the element types
the kernels consume (float32, bfloat16 bit patterns, OCP E4M3 codes plus
float32 per-token scales).  It holds none of the attention arithmetic; both
the HIP path (through the tests and the bench) and the CPU oracle read the
same arrays from here.

Draw order for one seed (numpy default_rng): sequence lengths (ragged cases
only), Q_nope, Q_rope, K_nope, K_rope, V, then the per-token magnitudes (fp8
cases only).  All draws are float32 standard normals, which keeps the large
cases at a few seconds of host time.
"""

from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np
import torch

E4M3_MAX = 448.0


@dataclasses.dataclass
class Inputs:
    """One attention problem in storage form (token-major THD layouts)."""

    dtype: str                      # "f32" | "bf16" | "fp8"
    q: np.ndarray                   # [T, Hq, Dn]  float32 | uint16 (bf16 bits) | uint8 (e4m3)
    k: np.ndarray                   # [T, Hkv, Dn] same element type as q
    v: np.ndarray                   # [T, Hkv, Dv] float32 (f32) | uint16 (bf16 bits)
    cu_seqlens: np.ndarray          # [B + 1] int32
    causal: bool
    q_rope: Optional[np.ndarray] = None   # [T, Hq, Dr]  bf16 bits (f32 for the f32 dtype)
    k_rope: Optional[np.ndarray] = None   # [T, Hkv, Dr]
    q_scale: Optional[np.ndarray] = None  # [T, Hq] float32 (fp8 only)
    k_scale: Optional[np.ndarray] = None  # [T, Hkv] float32 (fp8 only)
    softmax_scale: Optional[float] = None  # None: 1/sqrt(Dn + Dr)
    name: str = ""

    @property
    def total_tokens(self) -> int:
        return int(self.q.shape[0])

    @property
    def batch(self) -> int:
        return int(len(self.cu_seqlens) - 1)

    @property
    def num_heads(self) -> int:
        return int(self.q.shape[1])

    @property
    def num_kv_heads(self) -> int:
        return int(self.k.shape[1])

    @property
    def head_dim_nope(self) -> int:
        return int(self.q.shape[2])

    @property
    def head_dim_rope(self) -> int:
        return 0 if self.q_rope is None else int(self.q_rope.shape[2])

    @property
    def v_dim(self) -> int:
        return int(self.v.shape[2])

    @property
    def seqlens(self) -> np.ndarray:
        return np.diff(self.cu_seqlens.astype(np.int64))

    @property
    def max_seqlen(self) -> int:
        lens = self.seqlens
        return int(lens.max()) if len(lens) else 0


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def to_e4m3_per_row(x: np.ndarray):
    """float32 rows [T, H, D] -> (E4M3 codes uint8 [T, H, D], scales float32 [T, H]).

    scale = amax(|row|) / 448 (a zero row gets scale 1); codes are
    x / scale clamped to +-448 and rounded to nearest even in OCP E4M3.
    """
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    amax = t.abs().amax(dim=-1)
    scale = torch.where(amax > 0, amax / E4M3_MAX, torch.ones_like(amax))
    y = (t / scale[..., None]).clamp(-E4M3_MAX, E4M3_MAX)
    codes = y.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return codes, scale.numpy().astype(np.float32)


def _normal(rng, shape):
    return rng.standard_normal(size=shape, dtype=np.float32)


def make_inputs(*, dtype: str, seqlens, num_heads: int, num_kv_heads: int,
                head_dim_nope: int, v_dim: int, causal: bool,
                head_dim_rope: int = 0, seed: int = 0,
                softmax_scale: Optional[float] = None, name: str = "",
                rng: Optional[np.random.Generator] = None,
                fp8_magnitude_sigma: float = 0.5) -> Inputs:
    """Draw one problem: i.i.d. N(0,1) elements, packed along tokens.

    fp8: Q/K nope rows are N(0,1) vectors times a per-token lognormal(0,
    sigma) magnitude (one per token, shared by its heads), then quantised per
    (token, head) row; a rope part and V stay bfloat16.
    """
    if dtype not in ("f32", "bf16", "fp8"):
        raise ValueError(dtype)
    rng = np.random.default_rng(seed) if rng is None else rng
    lens = np.asarray(seqlens, dtype=np.int64)
    cu = np.zeros(len(lens) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lens)
    T = int(cu[-1])
    qn = _normal(rng, (T, num_heads, head_dim_nope))
    qr = _normal(rng, (T, num_heads, head_dim_rope)) if head_dim_rope else None
    kn = _normal(rng, (T, num_kv_heads, head_dim_nope))
    kr = _normal(rng, (T, num_kv_heads, head_dim_rope)) if head_dim_rope else None
    vv = _normal(rng, (T, num_kv_heads, v_dim))
    out = dict(dtype=dtype, cu_seqlens=cu, causal=bool(causal),
               softmax_scale=softmax_scale, name=name)
    if dtype == "f32":
        out.update(q=qn, k=kn, v=vv, q_rope=qr, k_rope=kr)
    elif dtype == "bf16":
        out.update(q=to_bf16_bits(qn), k=to_bf16_bits(kn), v=to_bf16_bits(vv),
                   q_rope=None if qr is None else to_bf16_bits(qr),
                   k_rope=None if kr is None else to_bf16_bits(kr))
    else:
        mq = rng.lognormal(0.0, fp8_magnitude_sigma, size=(T, 1, 1)).astype(np.float32)
        mk = rng.lognormal(0.0, fp8_magnitude_sigma, size=(T, 1, 1)).astype(np.float32)
        q8, qs = to_e4m3_per_row(qn * mq)
        k8, ks = to_e4m3_per_row(kn * mk)
        # a rope part stays bfloat16 (its own element type, unscaled)
        out.update(q=q8, k=k8, v=to_bf16_bits(vv), q_scale=qs, k_scale=ks,
                   q_rope=None if qr is None else to_bf16_bits(qr),
                   k_rope=None if kr is None else to_bf16_bits(kr))
    return Inputs(**out)


# The five workloads, by what they are.  "seqlens" is either a list or the
# string "ragged16", meaning 16 lengths drawn uniformly (inclusive) from
# [64, 8192] as the first draw of the seed.
WORKLOADS = {
    "fp32_b1_h2_s128_d64": dict(
        dtype="f32", seqlens=[128], num_heads=2, num_kv_heads=2,
        head_dim_nope=64, v_dim=64, causal=False),
    "bf16_causal_b4_h32_s4096_d128": dict(
        dtype="bf16", seqlens=[4096] * 4, num_heads=32, num_kv_heads=32,
        head_dim_nope=128, v_dim=128, causal=True),
    "bf16_varlen_gqa_causal_16seq_hq32_hkv8_d128": dict(
        dtype="bf16", seqlens="ragged16", num_heads=32, num_kv_heads=8,
        head_dim_nope=128, v_dim=128, causal=True),
    "bf16_nope128_rope64_causal_b2_h16_s8192": dict(
        dtype="bf16", seqlens=[8192] * 2, num_heads=16, num_kv_heads=16,
        head_dim_nope=128, head_dim_rope=64, v_dim=128, causal=True),
    "fp8_pertoken_causal_b8_h32_s4096_d128": dict(
        dtype="fp8", seqlens=[4096] * 8, num_heads=32, num_kv_heads=32,
        head_dim_nope=128, v_dim=128, causal=True),
}

WORKLOAD_ORDER = list(WORKLOADS)

# Workloads of the "next" rows: a long causal sequence over few heads, whose
# 256 query tiles (4 heads x 64) leave most compute units idle for most of
# the run unless the keys are split (split-KV).
EXTRA_WORKLOADS = {
    # fp8 nope + bf16 rope: the rope workload's shape with an 8-bit nope part
    "fp8_nope128_rope64_causal_b2_h16_s8192": dict(
        dtype="fp8", seqlens=[8192] * 2, num_heads=16, num_kv_heads=16,
        head_dim_nope=128, head_dim_rope=64, v_dim=128, causal=True),
    "bf16_causal_b1_h4_s16384_d128": dict(
        dtype="bf16", seqlens=[16384], num_heads=4, num_kv_heads=4,
        head_dim_nope=128, v_dim=128, causal=True),
    # the headline shape without the causal mask (the non-causal queue layout
    # and every query tile at full key length)
    "bf16_noncausal_b4_h32_s4096_d128": dict(
        dtype="bf16", seqlens=[4096] * 4, num_heads=32, num_kv_heads=32,
        head_dim_nope=128, v_dim=128, causal=False),
}


def ragged_lengths(rng: np.random.Generator, n: int = 16, lo: int = 64, hi: int = 8192):
    return rng.integers(lo, hi + 1, size=n)


def workload(name: str, seed: int = 0) -> Inputs:
    """The named workload's inputs, drawn from `seed`."""
    spec = dict(WORKLOADS[name] if name in WORKLOADS else EXTRA_WORKLOADS[name])
    rng = np.random.default_rng(seed)
    if spec["seqlens"] == "ragged16":
        spec["seqlens"] = ragged_lengths(rng)
    return make_inputs(**spec, rng=rng, name=name)


def attention_flops(inp: Inputs) -> float:
    """Metric FLOPs: 4 * Hq * Sq * Sk * D per sequence, halved when causal,
    with D = (Dqk + Dv) / 2 so that the split nope/rope depth counts the QK
    and PV products at their own depths."""
    d = (inp.head_dim_nope + inp.head_dim_rope + inp.v_dim) / 2.0
    lens = inp.seqlens.astype(np.float64)
    f = 4.0 * inp.num_heads * float(np.sum(lens * lens)) * d
    return f / 2.0 if inp.causal else f


def make_rows(shape, *, dtype: str = "bf16", seed: int = 0,
              magnitude_sigma: float = 1.0) -> np.ndarray:
    """Rows [..., D]: N(0,1) elements times one lognormal(0, sigma) magnitude
    per row, as float32 values (dtype "f32") or bfloat16 bit patterns
    ("bf16").  Inputs of the per-row fp8 quantiser."""
    if dtype not in ("f32", "bf16"):
        raise ValueError(dtype)
    rng = np.random.default_rng(seed)
    x = _normal(rng, tuple(shape))
    mag = rng.lognormal(0.0, magnitude_sigma, size=tuple(shape[:-1]) + (1,)).astype(np.float32)
    x = (x * mag).astype(np.float32)
    return x if dtype == "f32" else to_bf16_bits(x)


def make_partials(num_splits: int, total_tokens: int, num_heads: int, v_dim: int, *,
                  seed: int = 0, empty_fraction: float = 0.2):
    """Random partial results for the split merge: o_partial float32
    [n, T, H, Dv] ~ N(0,1) and lse_partial float32 [n, H, T] ~ N(0, 4), with
    about empty_fraction of the (split, head, token) entries set to an empty
    partial (o 0, lse -inf), including whole rows with every split empty."""
    rng = np.random.default_rng(seed)
    o = _normal(rng, (num_splits, total_tokens, num_heads, v_dim))
    lse = (_normal(rng, (num_splits, num_heads, total_tokens)) * 2.0).astype(np.float32)
    empty = rng.random((num_splits, num_heads, total_tokens)) < empty_fraction
    if total_tokens > 1:
        empty[:, :, total_tokens // 2] = True  # a row with every split empty
    lse[empty] = -np.inf
    o[np.transpose(empty, (0, 2, 1))] = 0.0
    return o, lse
