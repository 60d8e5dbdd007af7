"""Plain CPU oracle for split-KV attention and the log-sum-exp merge.

TEST INFRASTRUCTURE ONLY: imported by tests/, never by the product path.

Split-KV runs the attention of one query row over several disjoint key
ranges separately and merges the partial results afterwards.  The pages name
the knob (SM100AttentionSMem, comptime members: MiscMBarsType is built with
the config's splitk_partitions) and keep a per-row buffer for the running
softmax statistics (Methods: correction_smem); they print neither the
partial outputs nor the merge.
What is computed here is the plain definition:

partial result of row i over a key set K (the keys of range [lo, hi) that
the mask leaves visible to i):

    LSE_K(i) = log sum_{j in K} exp(S[i, j])
    O_K(i)   = sum_{j in K} exp(S[i, j] - LSE_K(i)) V[j]

and O_K = 0, LSE_K = -inf when K is empty (no visible key: the convention
the full oracle uses for an empty row).  Merging the partials of a partition
K_1 .. K_n of the visible keys gives the full result because the exponential
sums add:

    LSE(i) = log sum_s exp(LSE_s(i))
    O(i)   = sum_s exp(LSE_s(i) - LSE(i)) O_s(i)

(evaluated with the largest LSE_s factored out; all partials empty gives
O = 0, LSE = -inf).
"""

from __future__ import annotations

import numpy as np

from .attention import _check, default_softmax_scale


def mha_forward_key_range(q, k, v, cu_seqlens, causal, key_lo, key_hi,
                          softmax_scale=None, q_rope=None, k_rope=None):
    """Partial O [T, Hq, Dv] and LSE [Hq, T] (float64) of every query token
    over the keys j (indices local to its sequence) with
    key_lo[t] <= j < key_hi[t], intersected with the mask (j < L; causal:
    j <= i).  key_lo / key_hi are int arrays [T] (one range per query token,
    shared by its heads)."""
    q, k, v = (np.asarray(a, dtype=np.float64) for a in (q, k, v))
    if q_rope is not None:
        q_rope = np.asarray(q_rope, dtype=np.float64)
        k_rope = np.asarray(k_rope, dtype=np.float64)
    T, Hq, Hkv, cu = _check(q, k, v, cu_seqlens, q_rope, k_rope)
    lo_all = np.asarray(key_lo, dtype=np.int64)
    hi_all = np.asarray(key_hi, dtype=np.int64)
    dn = q.shape[2]
    dr = 0 if q_rope is None else q_rope.shape[2]
    sigma = default_softmax_scale(dn, dr) if softmax_scale is None else float(softmax_scale)
    group = Hq // Hkv
    o = np.full((T, Hq, v.shape[2]), np.nan)
    lse = np.full((Hq, T), np.nan)
    for b in range(len(cu) - 1):
        s0, s1 = int(cu[b]), int(cu[b + 1])
        L = s1 - s0
        if L == 0:
            continue
        i = np.arange(L)[:, None]
        j = np.arange(L)[None, :]
        visible = (j >= lo_all[s0:s1, None]) & (j < hi_all[s0:s1, None])
        if causal:
            visible &= j <= i
        empty = ~visible.any(axis=1)
        for h in range(Hq):
            g = h // group
            s = q[s0:s1, h] @ k[s0:s1, g].T
            if q_rope is not None:
                s = s + q_rope[s0:s1, h] @ k_rope[s0:s1, g].T
            s = np.where(visible, sigma * s, -np.inf)
            m = np.where(empty, 0.0, s.max(axis=1))
            p = np.exp(s - m[:, None])
            lsum = p.sum(axis=1)
            ob = (p @ v[s0:s1, g]) / np.where(empty, 1.0, lsum)[:, None]
            ob[empty] = 0.0
            o[s0:s1, h] = ob
            lse[h, s0:s1] = np.where(empty, -np.inf, m + np.log(np.where(empty, 1.0, lsum)))
    return o, lse


def merge_partials(o_parts, lse_parts):
    """o_parts [n, T, H, D], lse_parts [n, H, T] -> O [T, H, D], LSE [H, T]."""
    o_parts = np.asarray(o_parts, dtype=np.float64)
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    m = lse_parts.max(axis=0)                       # [H, T]
    empty = ~np.isfinite(m)
    m_safe = np.where(empty, 0.0, m)
    w = np.exp(lse_parts - m_safe[None])            # [n, H, T]; empty partials weigh 0
    total = w.sum(axis=0)
    lse = np.where(empty, -np.inf, m_safe + np.log(np.where(empty, 1.0, total)))
    wn = w / np.where(empty, 1.0, total)[None]      # exp(LSE_s - LSE)
    o = np.einsum("nht,nthd->thd", wn, o_parts)
    o[np.transpose(empty)] = 0.0
    return o, lse
