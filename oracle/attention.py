"""Plain float64 CPU oracle for the fused MHA forward pass.

TEST INFRASTRUCTURE ONLY: imported by tests/, by __graft_entry__.smoke() and
by bench.py's cpu_baseline leg, never by the product path.

What it computes is the definition of scaled-dot-product attention, evaluated
directly (full score matrix, ordinary softmax, float64 throughout):

    S  = sigma * (Q_nope K_nope^T + Q_rope K_rope^T)     per sequence, per head
    S[i, j] = -inf  where key j is hidden from query i   (causal: j > i)
    O  = softmax_rows(S) V
    LSE_i = log(sum_j exp(S[i, j]))                      natural log

The pages (three Modular API pages for an SM100 "FA4" attention kernel:
"SM100AttentionSMem", "TMAProducerPipeline" and "MHATileScheduler") do not
write this formula out; they name its pieces, and each function below cites
the one it follows:

* the split of Q and K into a "nope" part and a separately typed "rope" part
  (SM100AttentionSMem, Parameters: rope_dtype_; comptime members q_bytes,
  q_nope_bytes, q_rope_bytes);
* a per-token scale for Q and K (SM100AttentionSMem, Parameters:
  scale_dtype_; Methods q_scale_smem / k_scale_smem);
* per-batch sequence-length offsets, i.e. ragged batches packed along the
  token axis (MHATileScheduler, Required methods: get_current_work_info,
  parameter ValidLengthType);
* a per-row correction buffer for the running softmax statistics
  (SM100AttentionSMem, Methods: correction_smem) -- the online-softmax
  rescale.  The oracle does not use online softmax: it reaches the same
  result by the plain definition, which is what a flash-style kernel must
  equal up to rounding.

Readings where the pages are silent:
sigma defaults to 1/sqrt(Dn + Dr); the causal mask keeps key j for query i iff
j <= i in sequence-local indices (queries and keys share one length per
sequence); GQA maps query head h to KV head h // (Hq / Hkv); the rope parts are
already rotated data and only add their dot product to the score; under fp8,
Q and K are dequantised as code * scale[token, head] before the product.

Layouts (token-major, "THD"): q [T, Hq, Dn], k [T, Hkv, Dn], v [T, Hkv, Dv],
q_rope [T, Hq, Dr], k_rope [T, Hkv, Dr]; outputs O [T, Hq, Dv] and
LSE [Hq, T].  cu_seqlens is [B + 1] with cu_seqlens[0] = 0, nondecreasing.
"""

from __future__ import annotations

import math

import numpy as np

# Query rows per score block: bounds the float64 score matrix at
# ROW_CHUNK x L x 8 bytes (64 MiB at L = 8192).  This only splits the rows of
# an ordinary matrix product; every row is still computed in one piece.
ROW_CHUNK = 1024


def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> exact float64 values.

    bfloat16 is the upper half of an IEEE-754 binary32, so widening the
    pattern into the high 16 bits of a binary32 gives the value exactly.
    """
    bits = np.asarray(bits)
    if bits.dtype != np.uint16:
        raise TypeError("decode_bf16 expects uint16 bit patterns")
    wide = bits.astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):
        return wide.view(np.float32).astype(np.float64)


def decode_e4m3(codes: np.ndarray) -> np.ndarray:
    """OCP 8-bit float E4M3 ("fn": no infinities) codes (uint8) -> float64.

    Element type of Q and K under per-token scaling (SM100AttentionSMem,
    Parameters: qkv_dtype with scale_dtype_ set).  The pages do not name the
    8-bit format; this is the OCP E4M3 encoding: 1 sign bit, 4 exponent bits
    with bias 7, 3 mantissa bits; exponent 0 is subnormal (m/8 * 2^-6); the
    single pattern S.1111.111 is NaN; the largest finite value is 448.
    """
    codes = np.asarray(codes)
    if codes.dtype != np.uint8:
        raise TypeError("decode_e4m3 expects uint8 codes")
    c = codes.astype(np.int64)
    sign = np.where(c >> 7, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    normal = (1.0 + m / 8.0) * np.exp2((e - 7).astype(np.float64))
    subnormal = (m / 8.0) * 2.0 ** -6
    mag = np.where(e == 0, subnormal, normal)
    mag = np.where((e == 0xF) & ((c & 0x7) == 0x7), np.nan, mag)
    return sign * mag


def dequantize_per_token(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """fp8 codes [T, H, D] and scales [T, H] -> float64 values code * scale.

    One scale per (token, head) row (Q and K carry one scale per token:
    SM100AttentionSMem, Parameters: scale_dtype_; q_scale_smem holds BM of
    them per Q tile, k_scale_smem BN per K buffer).  The product of an E4M3
    value and a float32 scale is exact in float64.
    """
    vals = decode_e4m3(codes)
    s = np.asarray(scales, dtype=np.float64)
    if s.shape != vals.shape[:2]:
        raise ValueError("scales must be [T, H] for codes [T, H, D]")
    return vals * s[:, :, None]


def default_softmax_scale(head_dim_nope: int, head_dim_rope: int = 0) -> float:
    """sigma = 1/sqrt(Dn + Dr): the score is one dot product over the whole
    Q/K depth (nope plus rope), so the usual 1/sqrt(depth) uses both parts."""
    return 1.0 / math.sqrt(head_dim_nope + head_dim_rope)


def _check(q, k, v, cu_seqlens, q_rope, k_rope):
    for name, a in (("q", q), ("k", k), ("v", v)):
        if a.ndim != 3:
            raise ValueError(f"{name} must be [T, H, D]")
    T, Hq, _ = q.shape
    if k.shape[0] != T or v.shape[0] != T or k.shape[1] != v.shape[1]:
        raise ValueError("q, k, v must share T; k and v must share Hkv")
    Hkv = k.shape[1]
    if Hq % Hkv != 0:
        raise ValueError("num_heads must be a multiple of num_kv_heads")
    if (q_rope is None) != (k_rope is None):
        raise ValueError("q_rope and k_rope come together")
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    if cu[0] != 0 or np.any(np.diff(cu) < 0) or cu[-1] > T:
        raise ValueError("cu_seqlens must start at 0, be nondecreasing, end <= T")
    return T, Hq, Hkv, cu


def _head_block(qn, kn, vv, qr, kr, sigma, causal, row0):
    """Attention of query rows [row0, row0 + rows) of one sequence and head
    against all of that sequence's keys.  Returns (O rows, LSE rows)."""
    s = qn @ kn.T
    if qr is not None:
        s = s + qr @ kr.T
    s = sigma * s
    rows, L = s.shape
    if causal:
        qi = np.arange(row0, row0 + rows)[:, None]
        kj = np.arange(L)[None, :]
        s = np.where(kj <= qi, s, -np.inf)
    m = s.max(axis=1)
    empty = ~np.isfinite(m)
    m_safe = np.where(empty, 0.0, m)
    p = np.exp(s - m_safe[:, None])
    l = p.sum(axis=1)
    o = (p @ vv) / np.where(empty, 1.0, l)[:, None]
    o[empty] = 0.0
    lse = np.where(empty, -np.inf, m_safe + np.log(np.where(empty, 1.0, l)))
    return o, lse


def mha_forward(q, k, v, cu_seqlens, causal, softmax_scale=None,
                q_rope=None, k_rope=None):
    """O [T, Hq, Dv] and LSE [Hq, T] (float64) for every token of every
    sequence described by cu_seqlens.

    Inputs are already-decoded float64 arrays (see decode_bf16,
    dequantize_per_token).  Tokens outside [0, cu_seqlens[-1]) are left as NaN.
    """
    q, k, v = (np.asarray(a, dtype=np.float64) for a in (q, k, v))
    if q_rope is not None:
        q_rope = np.asarray(q_rope, dtype=np.float64)
        k_rope = np.asarray(k_rope, dtype=np.float64)
    T, Hq, Hkv, cu = _check(q, k, v, cu_seqlens, q_rope, k_rope)
    dn = q.shape[2]
    dr = 0 if q_rope is None else q_rope.shape[2]
    sigma = default_softmax_scale(dn, dr) if softmax_scale is None else float(softmax_scale)
    group = Hq // Hkv
    o = np.full((T, Hq, v.shape[2]), np.nan)
    lse = np.full((Hq, T), np.nan)
    for b in range(len(cu) - 1):
        s0, s1 = int(cu[b]), int(cu[b + 1])
        if s1 == s0:
            continue
        for h in range(Hq):
            g = h // group
            kn, vv = k[s0:s1, g], v[s0:s1, g]
            kr = None if k_rope is None else k_rope[s0:s1, g]
            for r0 in range(0, s1 - s0, ROW_CHUNK):
                r1 = min(r0 + ROW_CHUNK, s1 - s0)
                qn = q[s0 + r0:s0 + r1, h]
                qr = None if q_rope is None else q_rope[s0 + r0:s0 + r1, h]
                ob, lb = _head_block(qn, kn, vv, qr, kr, sigma, causal, r0)
                o[s0 + r0:s0 + r1, h] = ob
                lse[h, s0 + r0:s0 + r1] = lb
    return o, lse


def mha_forward_rows(q, k, v, cu_seqlens, causal, tokens, softmax_scale=None,
                     q_rope=None, k_rope=None):
    """The same definition, evaluated only for the query tokens listed in
    `tokens` (global token indices), for every query head.

    Returns O [len(tokens), Hq, Dv] and LSE [Hq, len(tokens)].  Used to check
    outputs at sizes where the full oracle would take too long: each row needs
    only its own sequence's keys.
    """
    q, k, v = (np.asarray(a) for a in (q, k, v))
    T, Hq, Hkv, cu = _check(q, k, v, cu_seqlens, q_rope, k_rope)
    dn = q.shape[2]
    dr = 0 if q_rope is None else q_rope.shape[2]
    sigma = default_softmax_scale(dn, dr) if softmax_scale is None else float(softmax_scale)
    group = Hq // Hkv
    tokens = np.asarray(tokens, dtype=np.int64)
    o = np.empty((len(tokens), Hq, v.shape[2]))
    lse = np.empty((Hq, len(tokens)))
    for n, t in enumerate(tokens):
        b = int(np.searchsorted(cu, t, side="right")) - 1
        if b < 0 or b >= len(cu) - 1 or not (cu[b] <= t < cu[b + 1]):
            raise ValueError(f"token {t} lies in no sequence")
        s0, s1 = int(cu[b]), int(cu[b + 1])
        i = int(t) - s0
        for h in range(Hq):
            g = h // group
            qn = np.asarray(q[t, h], dtype=np.float64)[None, :]
            kn = np.asarray(k[s0:s1, g], dtype=np.float64)
            vv = np.asarray(v[s0:s1, g], dtype=np.float64)
            qr = kr = None
            if q_rope is not None:
                qr = np.asarray(q_rope[t, h], dtype=np.float64)[None, :]
                kr = np.asarray(k_rope[s0:s1, g], dtype=np.float64)
            ob, lb = _head_block(qn, kn, vv, qr, kr, sigma, causal, i)
            o[n, h] = ob[0]
            lse[h, n] = lb[0]
    return o, lse
