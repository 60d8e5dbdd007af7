"""Pins for the CPU oracle: each test ties it to something other than itself.

* element decoders: every bf16 pattern and every E4M3 code against torch's own
  conversions, plus format facts of OCP E4M3 (max 448, min normal 2^-6, min
  subnormal 2^-9, NaN pattern);
* brute force: pure-Python scalar loops (math.exp / math.fsum, no max shift)
  on tiny inputs, covering causal and not, GQA ratios 1/2/4, the nope/rope
  split and ragged batches with empty sequences;
* a library special case: torch's float64 CPU flash-attention op (output and
  log-sum-exp) on the fp32 dense workload's shape;
* closed forms: Q = 0, constant V, causal row 0, one-token sequences;
* invariants: key shift, joint K/V permutation, softmax rows summing to one
  (V = identity), O-LSE consistency;
* reductions: GQA = repeated-KV MHA, ragged = per-sequence runs,
  nope/rope = concatenated depth, fp8 = attention on dequantised values;
* mutants: planted mistakes in a copy of the oracle's block routine fail the
  brute-force pin.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from oracle import attention as oatt
from mha_inputs import make_inputs, to_e4m3_per_row


def rand(rng, *shape):
    return rng.standard_normal(shape)


# ---------------------------------------------------------------- decoders

def test_decode_bf16_all_patterns():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ours = oracle.decode_bf16(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])


def test_decode_e4m3_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.decode_e4m3(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])


def test_decode_e4m3_format_facts():
    d = lambda c: float(oracle.decode_e4m3(np.array([c], dtype=np.uint8))[0])
    assert d(0x7E) == 448.0            # largest finite: 1.75 * 2^8
    assert d(0xFE) == -448.0
    assert d(0x38) == 1.0              # exponent field 7 = bias
    assert d(0xB8) == -1.0
    assert d(0x08) == 2.0 ** -6        # smallest normal
    assert d(0x01) == 2.0 ** -9        # smallest subnormal
    assert d(0x07) == 7 * 2.0 ** -9    # largest subnormal
    assert d(0x00) == 0.0 and math.copysign(1.0, d(0x80)) == -1.0
    assert math.isnan(d(0x7F)) and math.isnan(d(0xFF))
    # no infinities in this encoding
    assert np.all(np.isfinite(oracle.decode_e4m3(np.arange(0x7F, dtype=np.uint8))))


def test_dequantize_per_token_matches_codes_times_scale():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((5, 3, 16)).astype(np.float32) * 7
    codes, scales = to_e4m3_per_row(x)
    ours = oracle.dequantize_per_token(codes, scales)
    ref = (torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64)
           * torch.from_numpy(scales).to(torch.float64)[:, :, None]).numpy()
    assert np.array_equal(ours, ref)
    # per-row amax maps to the format maximum
    assert np.allclose(np.abs(ours).max(-1), np.abs(x).max(-1), rtol=1 / 16)


# ------------------------------------------------------------- brute force

def brute_force(q, k, v, cu, causal, sigma, qr=None, kr=None):
    """Scalar loops: S_ij, then exp(S_ij) / sum_k exp(S_ik), no max shift."""
    T, Hq, _ = q.shape
    Hkv = k.shape[1]
    Dv = v.shape[2]
    o = np.full((T, Hq, Dv), np.nan)
    lse = np.full((Hq, T), np.nan)
    for b in range(len(cu) - 1):
        s0, s1 = int(cu[b]), int(cu[b + 1])
        for h in range(Hq):
            g = (h * Hkv) // Hq
            for i in range(s1 - s0):
                ws = []
                for j in range(s1 - s0):
                    if causal and j > i:
                        continue
                    dot = math.fsum(float(q[s0 + i, h, d]) * float(k[s0 + j, g, d])
                                    for d in range(q.shape[2]))
                    if qr is not None:
                        dot += math.fsum(float(qr[s0 + i, h, d]) * float(kr[s0 + j, g, d])
                                         for d in range(qr.shape[2]))
                    ws.append((j, math.exp(sigma * dot)))
                z = math.fsum(w for _, w in ws)
                lse[h, s0 + i] = math.log(z)
                for c in range(Dv):
                    o[s0 + i, h, c] = math.fsum(w * float(v[s0 + j, g, c]) for j, w in ws) / z
    return o, lse


BRUTE_CASES = [
    # (lengths, Hq, Hkv, Dn, Dr, Dv, causal)
    ([5], 1, 1, 4, 0, 3, False),
    ([5], 1, 1, 4, 0, 3, True),
    ([7], 4, 2, 3, 0, 4, True),
    ([6], 4, 1, 4, 0, 2, False),
    ([6], 2, 2, 3, 2, 3, True),
    ([0, 1, 3, 8], 2, 1, 4, 0, 3, True),
    ([3, 0, 5], 4, 4, 2, 2, 2, False),
]


@pytest.mark.parametrize("case", BRUTE_CASES)
def test_oracle_matches_brute_force(case):
    lens, Hq, Hkv, Dn, Dr, Dv, causal = case
    rng = np.random.default_rng(11)
    T = sum(lens)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    q, k, v = rand(rng, T, Hq, Dn), rand(rng, T, Hkv, Dn), rand(rng, T, Hkv, Dv)
    qr = kr = None
    if Dr:
        qr, kr = rand(rng, T, Hq, Dr), rand(rng, T, Hkv, Dr)
    sigma = 1.0 / math.sqrt(Dn + Dr)
    o, lse = oracle.mha_forward(q, k, v, cu, causal, q_rope=qr, k_rope=kr)
    ob, lb = brute_force(q, k, v, cu, causal, sigma, qr, kr)
    assert np.allclose(o, ob, atol=1e-12, rtol=0, equal_nan=True)
    assert np.allclose(lse, lb, atol=1e-12, rtol=0, equal_nan=True)


# --------------------------------------------------------- library special case

@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("hq,hkv", [(2, 2), (4, 1)])
def test_oracle_matches_torch_flash_cpu(causal, hq, hkv):
    # torch's CPU flash-attention op returns output and natural-log LSE;
    # at the fp32 dense workload's shape (S = 128, D = 64).
    rng = np.random.default_rng(5)
    S, D = 128, 64
    q, k, v = rand(rng, S, hq, D), rand(rng, S, hkv, D), rand(rng, S, hkv, D)
    o, lse = oracle.mha_forward(q, k, v, np.array([0, S]), causal)
    tq = torch.from_numpy(q).permute(1, 0, 2)[None]
    rep = hq // hkv
    tk = torch.from_numpy(k).permute(1, 0, 2).repeat_interleave(rep, 0)[None]
    tv = torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(rep, 0)[None]
    to, tl = torch.ops.aten._scaled_dot_product_flash_attention_for_cpu(
        tq.contiguous(), tk.contiguous(), tv.contiguous(), 0.0, causal)
    assert np.allclose(o, to[0].permute(1, 0, 2).numpy(), atol=1e-12, rtol=0)
    assert np.allclose(lse, tl[0].numpy(), atol=1e-12, rtol=0)


def test_oracle_gqa_matches_torch_sdpa_enable_gqa():
    rng = np.random.default_rng(6)
    S, D, hq, hkv = 33, 16, 8, 2
    q, k, v = rand(rng, S, hq, D), rand(rng, S, hkv, D), rand(rng, S, hkv, D)
    o, _ = oracle.mha_forward(q, k, v, np.array([0, S]), True)
    t = lambda a: torch.from_numpy(a).permute(1, 0, 2)[None]
    ref = torch.nn.functional.scaled_dot_product_attention(
        t(q), t(k), t(v), is_causal=True, enable_gqa=True)
    assert np.allclose(o, ref[0].permute(1, 0, 2).numpy(), atol=1e-12, rtol=0)


# ------------------------------------------------------------- closed forms

@pytest.mark.parametrize("causal", [False, True])
def test_zero_query_gives_mean_of_visible_values(causal):
    rng = np.random.default_rng(7)
    L, H, D, Dv = 9, 2, 4, 3
    q = np.zeros((L, H, D))
    k, v = rand(rng, L, H, D), rand(rng, L, H, Dv)
    o, lse = oracle.mha_forward(q, k, v, np.array([0, L]), causal)
    for i in range(L):
        n = i + 1 if causal else L
        assert np.allclose(o[i], v[:n].mean(axis=0), atol=1e-14)
        assert np.allclose(lse[:, i], math.log(n), atol=1e-14)


def test_constant_value_rows_pass_through():
    rng = np.random.default_rng(8)
    L, H, D = 12, 3, 5
    c = rng.standard_normal((1, H, 4))
    v = np.repeat(c, L, axis=0)
    for causal in (False, True):
        o, _ = oracle.mha_forward(rand(rng, L, H, D), rand(rng, L, H, D), v,
                                  np.array([0, L]), causal)
        assert np.allclose(o, v, atol=1e-14)


def test_causal_row_zero_is_first_value():
    rng = np.random.default_rng(9)
    lens = [4, 1, 6]
    T = sum(lens)
    cu = np.array([0, 4, 5, 11])
    q, k, v = rand(rng, T, 2, 8), rand(rng, T, 2, 8), rand(rng, T, 2, 5)
    o, lse = oracle.mha_forward(q, k, v, cu, True)
    sigma = 1 / math.sqrt(8)
    for s in cu[:-1]:
        assert np.allclose(o[s], v[s], atol=1e-15)
        for h in range(2):
            assert lse[h, s] == pytest.approx(sigma * float(q[s, h] @ k[s, h]), abs=1e-14)
    # a one-token sequence is row zero even without a causal mask
    o2, lse2 = oracle.mha_forward(q, k, v, cu, False)
    assert np.allclose(o2[4], v[4], atol=1e-15)


# --------------------------------------------------------------- invariants

def test_key_shift_moves_lse_only():
    rng = np.random.default_rng(10)
    L, H, D = 10, 2, 6
    q, k, v = rand(rng, L, H, D), rand(rng, L, H, D), rand(rng, L, H, 3)
    u = rng.standard_normal((1, H, D))
    sigma = 1 / math.sqrt(D)
    for causal in (False, True):
        o1, l1 = oracle.mha_forward(q, k, v, np.array([0, L]), causal)
        o2, l2 = oracle.mha_forward(q, k + u, v, np.array([0, L]), causal)
        assert np.allclose(o1, o2, atol=1e-12)
        shift = sigma * np.einsum("thd,hd->ht", q, u[0])
        assert np.allclose(l2 - l1, shift, atol=1e-12)


def test_joint_kv_permutation_and_query_permutation():
    rng = np.random.default_rng(12)
    L, H, D = 11, 2, 5
    q, k, v = rand(rng, L, H, D), rand(rng, L, H, D), rand(rng, L, H, 4)
    cu = np.array([0, L])
    o, lse = oracle.mha_forward(q, k, v, cu, False)
    p = rng.permutation(L)
    o2, lse2 = oracle.mha_forward(q, k[p], v[p], cu, False)
    assert np.allclose(o, o2, atol=1e-12) and np.allclose(lse, lse2, atol=1e-12)
    o3, lse3 = oracle.mha_forward(q[p], k, v, cu, False)
    assert np.allclose(o3, o[p], atol=1e-12) and np.allclose(lse3, lse[:, p], atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_softmax_rows_sum_to_one(causal):
    # with V = identity the output rows are the probability rows themselves
    rng = np.random.default_rng(13)
    L, H, D = 8, 2, 4
    v = np.repeat(np.eye(L)[:, None, :], H, axis=1)
    o, _ = oracle.mha_forward(rand(rng, L, H, D), rand(rng, L, H, D), v,
                              np.array([0, L]), causal)
    assert np.allclose(o.sum(axis=2), 1.0, atol=1e-14)
    assert np.all(o >= 0)
    if causal:
        assert np.all(np.triu(o[:, 0, :], 1) == 0)


def test_output_consistent_with_lse():
    rng = np.random.default_rng(14)
    L, H, D = 9, 1, 4
    q, k, v = rand(rng, L, H, D), rand(rng, L, H, D), rand(rng, L, H, 3)
    sigma = 1 / math.sqrt(D)
    o, lse = oracle.mha_forward(q, k, v, np.array([0, L]), True)
    for i in range(L):
        w = np.array([math.exp(sigma * float(q[i, 0] @ k[j, 0]) - lse[0, i])
                      for j in range(i + 1)])
        assert math.isclose(w.sum(), 1.0, abs_tol=1e-13)
        assert np.allclose(w @ v[: i + 1, 0], o[i, 0], atol=1e-13)


# --------------------------------------------------------------- reductions

def test_gqa_equals_mha_with_repeated_kv():
    rng = np.random.default_rng(15)
    L, Hq, Hkv, D = 13, 8, 2, 4
    q, k, v = rand(rng, L, Hq, D), rand(rng, L, Hkv, D), rand(rng, L, Hkv, 5)
    cu = np.array([0, L])
    o, lse = oracle.mha_forward(q, k, v, cu, True)
    o2, lse2 = oracle.mha_forward(q, np.repeat(k, Hq // Hkv, axis=1),
                                  np.repeat(v, Hq // Hkv, axis=1), cu, True)
    assert np.allclose(o, o2, atol=1e-14) and np.allclose(lse, lse2, atol=1e-14)


def test_ragged_equals_per_sequence_runs():
    rng = np.random.default_rng(16)
    lens = [3, 0, 7, 1, 5]
    cu = np.concatenate([[0], np.cumsum(lens)])
    T = cu[-1]
    q, k, v = rand(rng, T, 2, 4), rand(rng, T, 2, 4), rand(rng, T, 2, 3)
    o, lse = oracle.mha_forward(q, k, v, cu, True)
    for b in range(len(lens)):
        s0, s1 = cu[b], cu[b + 1]
        if s1 == s0:
            continue
        ob, lb = oracle.mha_forward(q[s0:s1], k[s0:s1], v[s0:s1], np.array([0, s1 - s0]), True)
        assert np.allclose(o[s0:s1], ob, atol=1e-14)
        assert np.allclose(lse[:, s0:s1], lb, atol=1e-14)


def test_nope_rope_equals_concatenated_depth():
    rng = np.random.default_rng(17)
    L, H, Dn, Dr = 10, 2, 6, 3
    qn, kn = rand(rng, L, H, Dn), rand(rng, L, H, Dn)
    qr, kr = rand(rng, L, H, Dr), rand(rng, L, H, Dr)
    v = rand(rng, L, H, 4)
    cu = np.array([0, L])
    o, lse = oracle.mha_forward(qn, kn, v, cu, True, q_rope=qr, k_rope=kr)
    o2, lse2 = oracle.mha_forward(np.concatenate([qn, qr], 2), np.concatenate([kn, kr], 2),
                                  v, cu, True)
    assert np.allclose(o, o2, atol=1e-13) and np.allclose(lse, lse2, atol=1e-13)


def test_fp8_equals_attention_on_dequantised_values():
    inp = make_inputs(dtype="fp8", seqlens=[17, 5], num_heads=2, num_kv_heads=2,
                      head_dim_nope=16, v_dim=8, causal=True, seed=2)
    q = oracle.dequantize_per_token(inp.q, inp.q_scale)
    k = oracle.dequantize_per_token(inp.k, inp.k_scale)
    v = oracle.decode_bf16(inp.v)
    o, lse = oracle.mha_forward(q, k, v, inp.cu_seqlens, True)
    tq = (torch.from_numpy(inp.q).view(torch.float8_e4m3fn).double()
          * torch.from_numpy(inp.q_scale).double()[..., None]).numpy()
    tk = (torch.from_numpy(inp.k).view(torch.float8_e4m3fn).double()
          * torch.from_numpy(inp.k_scale).double()[..., None]).numpy()
    ob, lb = brute_force(tq, tk, v, inp.cu_seqlens, True, 1 / 4.0)
    assert np.allclose(o, ob, atol=1e-12) and np.allclose(lse, lb, atol=1e-12)


def test_fp8_nope_bf16_rope_scale_covers_the_nope_part_only():
    # reading of the mixed split: the per-token scales multiply the nope
    # product only; the rope part adds its bf16 dot product unscaled
    inp = make_inputs(dtype="fp8", seqlens=[11, 4], num_heads=2, num_kv_heads=1,
                      head_dim_nope=16, head_dim_rope=8, v_dim=8, causal=True, seed=4)
    q = oracle.dequantize_per_token(inp.q, inp.q_scale)
    k = oracle.dequantize_per_token(inp.k, inp.k_scale)
    qr, kr = oracle.decode_bf16(inp.q_rope), oracle.decode_bf16(inp.k_rope)
    v = oracle.decode_bf16(inp.v)
    o, lse = oracle.mha_forward(q, k, v, inp.cu_seqlens, True, q_rope=qr, k_rope=kr)
    tq = (torch.from_numpy(inp.q).view(torch.float8_e4m3fn).double()
          * torch.from_numpy(inp.q_scale).double()[..., None]).numpy()
    tk = (torch.from_numpy(inp.k).view(torch.float8_e4m3fn).double()
          * torch.from_numpy(inp.k_scale).double()[..., None]).numpy()
    ob, lb = brute_force(tq, tk, v, inp.cu_seqlens, True, 1 / math.sqrt(24.0), qr, kr)
    assert np.allclose(o, ob, atol=1e-12) and np.allclose(lse, lb, atol=1e-12)
    # the rope part really is unscaled: scaling it by q_scale changes the result
    ob2, _ = brute_force(tq, tk, v, inp.cu_seqlens, True, 1 / math.sqrt(24.0),
                         qr * inp.q_scale[..., None], kr)
    assert not np.allclose(o, ob2, atol=1e-6)


def test_rows_entry_matches_full_oracle():
    rng = np.random.default_rng(18)
    lens = [6, 9]
    cu = np.array([0, 6, 15])
    q, k, v = rand(rng, 15, 4, 4), rand(rng, 15, 2, 4), rand(rng, 15, 2, 3)
    qr, kr = rand(rng, 15, 4, 2), rand(rng, 15, 2, 2)
    o, lse = oracle.mha_forward(q, k, v, cu, True, q_rope=qr, k_rope=kr)
    toks = [0, 5, 6, 11, 14]
    o2, lse2 = oracle.mha_forward_rows(q, k, v, cu, True, toks, q_rope=qr, k_rope=kr)
    assert np.allclose(o2, o[toks], atol=1e-14)
    assert np.allclose(lse2, lse[:, toks], atol=1e-14)


# ------------------------------------------------------------------ mutants

def _mut_drop_rope(qn, kn, vv, qr, kr, sigma, causal, row0):
    return ORIG_BLOCK(qn, kn, vv, None, None, sigma, causal, row0)


def _mut_strict_causal(qn, kn, vv, qr, kr, sigma, causal, row0):
    # hides the diagonal: shifts the query index by one
    return ORIG_BLOCK(qn, kn, vv, qr, kr, sigma, causal, row0 - 1 if causal else row0)


def _mut_lse_log2(qn, kn, vv, qr, kr, sigma, causal, row0):
    o, lse = ORIG_BLOCK(qn, kn, vv, qr, kr, sigma, causal, row0)
    return o, lse / math.log(2.0)


def _mut_no_sigma(qn, kn, vv, qr, kr, sigma, causal, row0):
    return ORIG_BLOCK(qn, kn, vv, qr, kr, 1.0, causal, row0)


def _mut_key_order(qn, kn, vv, qr, kr, sigma, causal, row0):
    # pairs each score with the wrong value row (a transposed/flipped operand)
    return ORIG_BLOCK(qn, kn, vv[::-1].copy(), qr, kr, sigma, causal, row0)


ORIG_BLOCK = oatt._head_block


@pytest.mark.parametrize("mutant", [_mut_drop_rope, _mut_strict_causal, _mut_lse_log2,
                                    _mut_no_sigma, _mut_key_order])
def test_planted_mistakes_fail_brute_force_pin(mutant, monkeypatch):
    monkeypatch.setattr(oatt, "_head_block", mutant)
    lens, Hq, Hkv, Dn, Dr, Dv, causal = ([6], 2, 2, 3, 2, 3, True)
    rng = np.random.default_rng(11)
    T = sum(lens)
    cu = np.array([0, T])
    q, k, v = rand(rng, T, Hq, Dn), rand(rng, T, Hkv, Dn), rand(rng, T, Hkv, Dv)
    qr, kr = rand(rng, T, Hq, Dr), rand(rng, T, Hkv, Dr)
    o, lse = oracle.mha_forward(q, k, v, cu, causal, q_rope=qr, k_rope=kr)
    ob, lb = brute_force(q, k, v, cu, causal, 1 / math.sqrt(Dn + Dr), qr, kr)
    agree = (np.allclose(o, ob, atol=1e-9, equal_nan=True)
             and np.allclose(lse, lb, atol=1e-9, equal_nan=True))
    assert not agree
