"""Helpers shared by the GPU tests: move seeded inputs to the device, run the
HIP path through the binding, and evaluate the oracle on the same inputs."""

from __future__ import annotations

import numpy as np
import torch

import oracle
from mha_inputs import Inputs

TOL_O = {"f32": 1e-4, "bf16": 2e-2, "fp8": 6e-2}
TOL_LSE = 1e-3


def device_tensors(inp: Inputs, device="cuda:0"):
    def bits(a, dt):
        if a is None:
            return None
        if dt == "bf16":
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)
        if dt == "fp8":
            return torch.from_numpy(a).view(torch.float8_e4m3fn).to(device)
        return torch.from_numpy(a).to(device)

    qk_dt = inp.dtype
    v_dt = "f32" if inp.dtype == "f32" else "bf16"
    return dict(
        q=bits(inp.q, qk_dt), k=bits(inp.k, qk_dt), v=bits(inp.v, v_dt),
        q_rope=bits(inp.q_rope, v_dt), k_rope=bits(inp.k_rope, v_dt),
        q_scale=None if inp.q_scale is None else torch.from_numpy(inp.q_scale).to(device),
        k_scale=None if inp.k_scale is None else torch.from_numpy(inp.k_scale).to(device),
        cu_seqlens=torch.from_numpy(inp.cu_seqlens).to(device),
    )


def run_gpu(inp: Inputs, device="cuda:0", tensors=None, fp8_fast_accum=False):
    from head_attention_forward_fa_amd import mha_fwd
    t = tensors or device_tensors(inp, device)
    o, lse = mha_fwd(t["q"], t["k"], t["v"], causal=inp.causal, cu_seqlens=t["cu_seqlens"],
                     max_seqlen=inp.max_seqlen, q_rope=t["q_rope"], k_rope=t["k_rope"],
                     q_scale=t["q_scale"], k_scale=t["k_scale"],
                     softmax_scale=inp.softmax_scale, fp8_fast_accum=fp8_fast_accum)
    torch.cuda.synchronize()
    return o, lse


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def decoded(inp: Inputs, lo: int = 0, hi: int | None = None):
    """Oracle-side float64 values of tokens [lo, hi)."""
    hi = inp.total_tokens if hi is None else hi
    sl = slice(lo, hi)
    if inp.dtype == "f32":
        dec = lambda a: None if a is None else a[sl].astype(np.float64)
        q, k = dec(inp.q), dec(inp.k)
        v, qr, kr = dec(inp.v), dec(inp.q_rope), dec(inp.k_rope)
    else:
        dec = lambda a: None if a is None else oracle.decode_bf16(a[sl])
        if inp.dtype == "fp8":
            q = oracle.dequantize_per_token(inp.q[sl], inp.q_scale[sl])
            k = oracle.dequantize_per_token(inp.k[sl], inp.k_scale[sl])
        else:
            q, k = dec(inp.q), dec(inp.k)
        v, qr, kr = dec(inp.v), dec(inp.q_rope), dec(inp.k_rope)
    return q, k, v, qr, kr


def oracle_full(inp: Inputs):
    q, k, v, qr, kr = decoded(inp)
    return oracle.mha_forward(q, k, v, inp.cu_seqlens, inp.causal, inp.softmax_scale,
                              q_rope=qr, k_rope=kr)


def oracle_rows(inp: Inputs, tokens):
    """Oracle O [n, Hq, Dv] and LSE [Hq, n] at the given global tokens,
    decoding only the sequences that hold them."""
    tokens = np.asarray(tokens, dtype=np.int64)
    cu = inp.cu_seqlens.astype(np.int64)
    o = np.empty((len(tokens), inp.num_heads, inp.v_dim))
    lse = np.empty((inp.num_heads, len(tokens)))
    seq = np.searchsorted(cu, tokens, side="right") - 1
    for b in np.unique(seq):
        s0, s1 = int(cu[b]), int(cu[b + 1])
        idx = np.nonzero(seq == b)[0]
        q, k, v, qr, kr = decoded(inp, s0, s1)
        ob, lb = oracle.mha_forward_rows(q, k, v, np.array([0, s1 - s0]), inp.causal,
                                         tokens[idx] - s0, inp.softmax_scale,
                                         q_rope=qr, k_rope=kr)
        o[idx] = ob
        lse[:, idx] = lb
    return o, lse


def sample_tokens(inp: Inputs, n_random: int = 256, seed: int = 1):
    """First, last and tile-boundary rows of every sequence (the first and
    last row of every 256-row query tile, so that a work item that wrote the
    wrong tile or not at all shows), plus random ones."""
    cu = inp.cu_seqlens.astype(np.int64)
    rng = np.random.default_rng(seed)
    toks = set()
    for b in range(len(cu) - 1):
        s0, s1 = int(cu[b]), int(cu[b + 1])
        if s1 == s0:
            continue
        for i in (0, 1, 31, 32, 63, 64, 127, 128, 255, 256, 257, 4095, 4096,
                  s1 - s0 - 2, s1 - s0 - 1):
            if 0 <= i < s1 - s0:
                toks.add(s0 + i)
        for t0 in range(0, s1 - s0, 256):
            toks.add(s0 + t0)
            toks.add(s0 + min(t0 + 255, s1 - s0 - 1))
    if inp.total_tokens:
        toks.update(int(x) for x in rng.integers(0, inp.total_tokens, n_random))
    return np.array(sorted(toks), dtype=np.int64)


def max_abs(a, b):
    return float(np.max(np.abs(np.asarray(a) - np.asarray(b)))) if np.size(a) else 0.0


def split_key_ranges(cu_seqlens, causal: bool, num_splits: int, block_m: int = 256,
                     block_n: int = 64):
    """lo, hi int arrays [num_splits, T]: the key range (local indices) of
    each split for every query token, by the rule mha_fwd_splitkv documents:
    a query tile of block_m rows sees nb = ceil(n / block_n) key blocks (n =
    min(L, block_m (qt + 1)) causal, else L); split s holds blocks
    [s p, min((s + 1) p, nb)), p = ceil(nb / num_splits)."""
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    T = int(cu[-1])
    lo = np.zeros((num_splits, T), np.int64)
    hi = np.zeros((num_splits, T), np.int64)
    for b in range(len(cu) - 1):
        L = int(cu[b + 1] - cu[b])
        for i in range(L):
            qt = i // block_m
            n = min(L, block_m * (qt + 1)) if causal else L
            nb = -(-n // block_n)
            p = -(-nb // num_splits)
            for s in range(num_splits):
                b0, b1 = min(nb, s * p), min(nb, (s + 1) * p)
                lo[s, cu[b] + i] = b0 * block_n
                hi[s, cu[b] + i] = b1 * block_n
    return lo, hi


def fast_accum_lse_bound(inp: Inputs, rel: float = 2.0 ** -12):
    """Per-row LSE error bound [Hq, T] for fp8 with the fp8 matrix
    instruction: that instruction's sum of products errs by up to about
    2^-13 of the sum of the products' magnitudes (measured on gfx950; rel
    doubles it for margin), so each score errs by at most
    rel * sigma * sum_d |q_d k_d| over the nope depth (the rope part runs on
    the bf16 instruction), and an LSE, a softmax-weighted mean of its row's
    scores to first order, by at most the largest of those over the visible
    keys."""
    q, k, _, _, _ = decoded(inp)
    cu = inp.cu_seqlens.astype(np.int64)
    group = inp.num_heads // inp.num_kv_heads
    sigma = (inp.softmax_scale if inp.softmax_scale
             else 1.0 / np.sqrt(inp.head_dim_nope + inp.head_dim_rope))
    bound = np.zeros((inp.num_heads, inp.total_tokens))
    for b in range(inp.batch):
        s0, s1 = int(cu[b]), int(cu[b + 1])
        if s1 == s0:
            continue
        for h in range(inp.num_heads):
            g = h // group
            m = np.abs(q[s0:s1, h]) @ np.abs(k[s0:s1, g]).T
            if inp.causal:
                m = np.tril(m)
            bound[h, s0:s1] = rel * sigma * m.max(axis=1)
    return bound
