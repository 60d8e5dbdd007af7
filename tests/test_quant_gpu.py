"""GPU per-row fp8 quantiser (mha_quantize_fp8) vs the oracle, bit for bit.

Codes and scales are integers / exact float32 results of the definition
(scale = amax / 448, code = nearest E4M3 of x / scale, ties to even), so the
comparison is exact: random rows of both input types and several widths with
a ragged last workgroup, rows built to hit every E4M3 midpoint (and the next
float on either side), zero rows, and the fp8 workload's Q at full size on
sampled rows.  End to end: Q and K quantised on the device drive the fp8
attention path to the same output as the same codes made on the host.
"""

import numpy as np
import pytest
import torch

import mha_inputs as mi
from oracle import quantize as oq

pytestmark = pytest.mark.gpu


def _dev(x: np.ndarray, dtype: str):
    if dtype == "bf16":
        return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(x).cuda()


def _oracle(x: np.ndarray, dtype: str):
    return oq.quantize_bf16_rows(x) if dtype == "bf16" else oq.quantize_rows(x)


def _quant(xd):
    from head_attention_forward_fa_amd import mha_quantize_fp8
    c, s = mha_quantize_fp8(xd)
    torch.cuda.synchronize()
    return c.cpu().numpy(), s.cpu().numpy()


def _assert_same(c, s, rc, rs, what):
    assert np.array_equal(s.view(np.uint32), rs.view(np.uint32)), f"{what}: scales differ"
    bad = np.argwhere(c != rc)
    assert bad.size == 0, f"{what}: {len(bad)} codes differ, first at {bad[0]}: {c[tuple(bad[0])]:#x} vs {rc[tuple(bad[0])]:#x}"


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("rows,cols", [(1, 8), (37, 64), (1000, 128), (333, 192), (65, 512),
                                       (5001, 128), (17, 136)])
def test_random_rows(dtype, rows, cols):
    x = mi.make_rows((rows, cols), dtype=dtype, seed=rows * 7 + cols)
    c, s = _quant(_dev(x, dtype))
    rc, rs = _oracle(x, dtype)
    _assert_same(c, s, rc, rs, f"{dtype} {rows}x{cols}")


def _midpoint_rows(dtype):
    vals, _ = oq.e4m3_table()
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)
    cand = [mids, -mids]
    if dtype == "f32":
        cand += [np.nextafter(mids, np.float32(1e9)), np.nextafter(mids, np.float32(0)),
                 -np.nextafter(mids, np.float32(1e9))]
    body = np.concatenate(cand).astype(np.float32)
    cols = 128
    per = cols - 1
    n = (len(body) + per - 1) // per
    body = np.concatenate([body, np.zeros(n * per - len(body), np.float32)])
    # first element 448 in every row: amax = 448, scale = 1, x / scale = x
    rows = np.concatenate([np.full((n, 1), 448.0, np.float32), body.reshape(n, per)], axis=1)
    rows = np.concatenate([rows, np.zeros((1, cols), np.float32)])  # and a zero row
    if dtype == "bf16":
        bits = mi.to_bf16_bits(rows)
        assert np.array_equal(oq.decode_bf16(bits), rows.astype(np.float64))  # exact in bf16
        return bits
    return rows


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_midpoints_ties_and_zero_rows(dtype):
    x = _midpoint_rows(dtype)
    c, s = _quant(_dev(x, dtype))
    rc, rs = _oracle(x, dtype)
    assert np.all(rs[:-1] == 1.0) and rs[-1] == 1.0 and np.all(rc[-1] == 0)
    _assert_same(c, s, rc, rs, f"{dtype} midpoints")


def _near_midpoint_rows():
    # quotients x / scale a few float32 ulps either side of every E4M3
    # midpoint, under scales that are not powers of two (and one below
    # 2^-100): the device's fast quotient (a reciprocal product, checked
    # against the midpoints) must agree with the IEEE division everywhere
    vals, _ = oq.e4m3_table()
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)
    mids = mids[mids > 0]
    rows = []
    for amax in (np.float32(448 * 1.2345678), np.float32(3.7), np.float32(0.0123),
                 np.float32(77.7), np.float32(2e-31)):
        scale = np.float32(amax / np.float32(448))
        for k in range(-6, 7):
            xs = (mids * scale).astype(np.float32)
            if k:
                step = np.float32(np.inf) if k > 0 else np.float32(0)
                for _ in range(abs(k)):
                    xs = np.nextafter(xs, step).astype(np.float32)
            xs = np.minimum(np.abs(xs), amax)
            body = np.concatenate([xs, -xs])
            per = 127
            n = (len(body) + per - 1) // per
            body = np.concatenate([body, np.zeros(n * per - len(body), np.float32)])
            rows.append(np.concatenate([np.full((n, 1), amax, np.float32),
                                        body.reshape(n, per)], axis=1))
    return np.concatenate(rows).astype(np.float32)


def test_near_midpoints_under_general_scales():
    x = _near_midpoint_rows()
    c, s = _quant(_dev(x, "f32"))
    rc, rs = _oracle(x, "f32")
    _assert_same(c, s, rc, rs, "near midpoints")


def test_full_size_fp8_workload_q_sampled_rows():
    # Q of the fp8 workload: 8 x 4096 tokens, 32 heads, D 128, bf16 rows
    T, H, D = 8 * 4096, 32, 128
    x = mi.make_rows((T, H, D), dtype="bf16", seed=11, magnitude_sigma=0.5)
    c, s = _quant(_dev(x, "bf16"))
    rng = np.random.default_rng(0)
    toks = np.unique(np.concatenate([[0, 1, T - 1], rng.integers(0, T, 512)]))
    rc, rs = _oracle(x[toks], "bf16")
    _assert_same(c[toks], s[toks], rc, rs, "full-size sampled")


def test_device_quantised_inputs_drive_the_fp8_path():
    from head_attention_forward_fa_amd import mha_fwd
    inp = mi.make_inputs(dtype="f32", seqlens=[300, 77], num_heads=4, num_kv_heads=2,
                         head_dim_nope=128, v_dim=128, causal=True, seed=5)
    qd, kd = torch.from_numpy(inp.q).cuda(), torch.from_numpy(inp.k).cuda()
    from head_attention_forward_fa_amd import mha_quantize_fp8
    qc, qs = mha_quantize_fp8(qd)
    kc, ks = mha_quantize_fp8(kd)
    hq, hqs = oq.quantize_rows(inp.q)
    hk, hks = oq.quantize_rows(inp.k)
    assert np.array_equal(qc.cpu().numpy(), hq) and np.array_equal(kc.cpu().numpy(), hk)
    v = torch.from_numpy(mi.to_bf16_bits(inp.v).view(np.int16)).view(torch.bfloat16).cuda()
    cu = torch.from_numpy(inp.cu_seqlens).cuda()
    o1, l1 = mha_fwd(qc.view(torch.float8_e4m3fn), kc.view(torch.float8_e4m3fn), v, causal=True,
                     cu_seqlens=cu, max_seqlen=300, q_scale=qs, k_scale=ks)
    o2, l2 = mha_fwd(torch.from_numpy(hq).cuda().view(torch.float8_e4m3fn),
                     torch.from_numpy(hk).cuda().view(torch.float8_e4m3fn), v, causal=True,
                     cu_seqlens=cu, max_seqlen=300, q_scale=torch.from_numpy(hqs).cuda(),
                     k_scale=torch.from_numpy(hks).cuda())
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
