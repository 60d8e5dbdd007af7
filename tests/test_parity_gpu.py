"""HIP path vs the float64 oracle, element by element, through the C ABI.

Small cases (seconds for the oracle) span several 256-row query tiles and
64-key blocks (enough of them to wrap the kernel's K and V rings) with ragged tails, GQA, empty sequences, the nope/rope split and
fp8; the five named workloads run at full size with the oracle evaluated on
sampled rows (first, last, tile-boundary and random tokens, every head).
Tolerances (max-abs): O 1e-4 fp32, 2e-2 bf16, 6e-2 fp8; LSE 1e-3.
"""

import numpy as np
import pytest
import torch

import mha_inputs as mi
from _util import (TOL_LSE, TOL_O, device_tensors, fast_accum_lse_bound, max_abs, oracle_full,
                   oracle_rows, run_gpu, sample_tokens, to_f64)

pytestmark = pytest.mark.gpu

SMALL = [
    # dtype, lengths, Hq, Hkv, Dn, Dr, Dv, causal
    ("bf16", [300], 4, 4, 128, 0, 128, True),
    ("bf16", [300], 4, 4, 128, 0, 128, False),
    ("bf16", [1, 129, 0, 517, 64], 8, 2, 128, 0, 128, True),
    ("bf16", [1, 129, 0, 517, 64], 8, 2, 128, 0, 128, False),
    ("bf16", [200, 77], 4, 1, 64, 0, 64, True),
    ("bf16", [200, 77], 4, 1, 64, 0, 64, False),
    ("bf16", [1100], 2, 2, 128, 0, 128, True),
    ("bf16", [1100, 31], 2, 1, 128, 0, 128, False),
    ("bf16", [333], 4, 4, 128, 64, 128, True),
    ("bf16", [650], 2, 2, 128, 64, 128, False),
    ("bf16", [190, 5], 4, 2, 128, 64, 128, False),
    ("fp8", [300, 50], 4, 4, 128, 0, 128, True),
    ("fp8", [300, 50], 4, 4, 128, 0, 128, False),
    ("fp8", [257], 8, 2, 128, 0, 128, True),
    ("fp8", [900], 2, 2, 128, 0, 128, True),
    ("fp8", [333, 20], 4, 4, 128, 64, 128, True),
    ("fp8", [650], 2, 1, 128, 64, 128, False),
    ("f32", [100, 3], 2, 2, 128, 0, 128, True),
    ("f32", [70], 2, 1, 128, 64, 128, True),
    ("f32", [130, 1], 2, 2, 64, 0, 64, True),
    ("f32", [130, 1], 2, 2, 64, 0, 64, False),
    ("f32", [300, 1, 0, 129, 64], 8, 2, 64, 0, 64, True),
    ("f32", [300, 1, 0, 129, 64], 8, 2, 64, 0, 64, False),
    ("f32", [517, 33], 4, 2, 128, 0, 128, False),
    ("f32", [260, 31], 2, 2, 128, 64, 128, False),
    # wide query-head groups: multi-query (one KV head) and 16 per KV head
    ("bf16", [333, 70], 32, 1, 128, 0, 128, True),
    ("bf16", [200], 64, 4, 64, 0, 64, False),
    ("fp8", [260], 16, 1, 128, 0, 128, True),
    ("bf16", [150], 16, 1, 128, 64, 128, True),
    # more items than workgroups (about 1 000 against 256): every workgroup
    # runs several items in a row, so whatever an item carries over to the
    # next (its Q fragments, the fp8 q_scale multiplier, the next item's
    # entry) is exercised
    ("fp8", [300, 257, 40, 512] * 8, 16, 4, 128, 0, 128, True),
    ("bf16", [300, 257, 40, 512] * 8, 16, 4, 128, 0, 128, True),
    ("bf16", [300, 257, 40, 512] * 8, 16, 16, 128, 64, 128, True),
    ("f32", [300, 257, 40, 512] * 4, 8, 2, 64, 0, 64, True),
]


def _check(inp, o, lse, ref_o, ref_lse, tokens=None):
    o64, lse64 = to_f64(o), to_f64(lse)
    if tokens is not None:
        o64, lse64 = o64[tokens], lse64[:, tokens]
    eo, el = max_abs(o64, ref_o), max_abs(lse64, ref_lse)
    assert np.all(np.isfinite(o64)) and np.all(np.isfinite(lse64))
    assert eo <= TOL_O[inp.dtype], f"{inp.name}: O max-abs {eo}"
    assert el <= TOL_LSE, f"{inp.name}: LSE max-abs {el}"
    return eo, el


def _case_id(c):
    lens = c[1] if len(c[1]) <= 6 else f"{len(c[1])}seq"
    return f"{c[0]}-{lens}-{c[2]}x{c[3]}-{c[4]}+{c[5]}-{c[6]}-{'c' if c[7] else 'nc'}"


@pytest.mark.parametrize("case", SMALL, ids=_case_id)
def test_small_cases_match_oracle(case):
    dt, lens, hq, hkv, dn, dr, dv, causal = case
    inp = mi.make_inputs(dtype=dt, seqlens=lens, num_heads=hq, num_kv_heads=hkv,
                         head_dim_nope=dn, head_dim_rope=dr, v_dim=dv, causal=causal,
                         seed=7, name=str(case))
    print("case", case, flush=True)
    o, lse = run_gpu(inp)
    ref_o, ref_lse = oracle_full(inp)
    _check(inp, o, lse, ref_o, ref_lse)


FAST = [
    # dtype, lengths, Hq, Hkv, Dn, Dr, Dv, causal
    ("fp8", [300, 50], 4, 4, 128, 0, 128, True),
    ("fp8", [257, 0, 129], 8, 2, 128, 0, 128, False),
    ("fp8", [333, 20], 4, 4, 128, 64, 128, True),
    ("fp8", [300, 257, 40, 512] * 4, 16, 4, 128, 0, 128, True),
]


@pytest.mark.parametrize("case", FAST, ids=_case_id)
def test_fp8_fast_accum_within_its_bound(case):
    """MHA_DTYPE_FP8_E4M3_FASTACC: O at the fp8 tolerance; LSE within the
    per-row bound that the fp8 matrix instruction's accumulation precision
    gives (fast_accum_lse_bound) plus the LSE tolerance."""
    dt, lens, hq, hkv, dn, dr, dv, causal = case
    inp = mi.make_inputs(dtype=dt, seqlens=lens, num_heads=hq, num_kv_heads=hkv,
                         head_dim_nope=dn, head_dim_rope=dr, v_dim=dv, causal=causal,
                         seed=7, name=str(case))
    print("fast-accum case", case, flush=True)
    o, lse = run_gpu(inp, fp8_fast_accum=True)
    ref_o, ref_lse = oracle_full(inp)
    o64, lse64 = to_f64(o), to_f64(lse)
    assert np.all(np.isfinite(o64)) and np.all(np.isfinite(lse64))
    assert max_abs(o64, ref_o) <= TOL_O["fp8"]
    err = np.abs(lse64 - ref_lse)
    bound = fast_accum_lse_bound(inp) + TOL_LSE
    assert np.all(err <= bound), f"worst excess {np.max(err - bound)}"


def test_fp32_dense_workload_full():
    inp = mi.workload("fp32_b1_h2_s128_d64")
    o, lse = run_gpu(inp)
    ref_o, ref_lse = oracle_full(inp)
    eo, el = _check(inp, o, lse, ref_o, ref_lse)
    print(f"fp32 workload: O err {eo:.3e}, LSE err {el:.3e}")


@pytest.mark.parametrize("name", mi.WORKLOAD_ORDER[1:] + list(mi.EXTRA_WORKLOADS))
def test_full_size_workloads_sampled(name):
    print("workload", name, flush=True)
    inp = mi.workload(name)
    o, lse = run_gpu(inp)
    # every row of every head is finite; sampled rows match the oracle
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(lse).all())
    toks = sample_tokens(inp)
    ref_o, ref_lse = oracle_rows(inp, toks)
    eo, el = _check(inp, o, lse, ref_o, ref_lse, tokens=toks)
    print(f"{name}: {len(toks)} tokens x {inp.num_heads} heads, O err {eo:.3e}, LSE err {el:.3e}")


@pytest.mark.parametrize("dtype,dn,dr,scale", [("bf16", 128, 0, 0.31), ("bf16", 128, 64, 0.02),
                                               ("fp8", 128, 0, 0.4), ("f32", 64, 0, 1.7)])
def test_explicit_softmax_scale(dtype, dn, dr, scale):
    """A softmax scale other than 1/sqrt(Dn + Dr) reaches every kernel (large
    scales sharpen the rows, small ones flatten them)."""
    inp = mi.make_inputs(dtype=dtype, seqlens=[300, 41], num_heads=4, num_kv_heads=2,
                         head_dim_nope=dn, head_dim_rope=dr, v_dim=dn, causal=True, seed=17,
                         softmax_scale=scale)
    print("scale", dtype, dn, dr, scale, flush=True)
    o, lse = run_gpu(inp)
    ref_o, ref_lse = oracle_full(inp)
    _check(inp, o, lse, ref_o, ref_lse)


@pytest.mark.parametrize("causal", [True, False], ids=["causal", "noncausal"])
def test_long_sequence_sampled(causal):
    """One sequence of 131 072 tokens (GQA 2 / 1, D 128): far past the
    configurations' lengths, so that token, block and table offsets run
    large; mha_fwd splits the keys of its few long items by itself.  Rows
    at the start, the end and around q-tile boundaries near the end, plus
    random ones, against the oracle."""
    S = 131072
    inp = mi.make_inputs(dtype="bf16", seqlens=[S], num_heads=2, num_kv_heads=1,
                         head_dim_nope=128, v_dim=128, causal=causal, seed=21)
    print("long sequence", S, "causal" if causal else "non-causal", flush=True)
    o, lse = run_gpu(inp)
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(lse).all())
    rng = np.random.default_rng(5)
    toks = {0, 1, 255, 256, S - 1, S - 2}
    for t0 in (S - 4 * 256, S - 2 * 256, S - 256):
        toks.update((t0 - 1, t0, t0 + 255))
    toks.update(int(x) for x in rng.integers(0, S, 24))
    toks = np.array(sorted(toks), dtype=np.int64)
    ref_o, ref_lse = oracle_rows(inp, toks)
    eo, el = _check(inp, o, lse, ref_o, ref_lse, tokens=toks)
    print(f"long sequence: {len(toks)} tokens x 2 heads, O err {eo:.3e}, LSE err {el:.3e}")


def test_dense_layout_equals_packed():
    inp = mi.make_inputs(dtype="bf16", seqlens=[256, 256], num_heads=4, num_kv_heads=2,
                         head_dim_nope=128, v_dim=128, causal=True, seed=3)
    from head_attention_forward_fa_amd import mha_fwd
    t = device_tensors(inp)
    o1, l1 = run_gpu(inp, tensors=t)
    r = lambda x: x.view(2, 256, *x.shape[1:])
    o2, l2 = mha_fwd(r(t["q"]), r(t["k"]), r(t["v"]), causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2.reshape_as(o1)) and torch.equal(l1, l2)


def test_repeat_calls_are_bitwise_identical():
    inp = mi.make_inputs(dtype="bf16", seqlens=[700, 33], num_heads=8, num_kv_heads=8,
                         head_dim_nope=128, v_dim=128, causal=True, seed=4)
    t = device_tensors(inp)
    o1, l1 = run_gpu(inp, tensors=t)
    o2, l2 = run_gpu(inp, tensors=t)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_kernel_events_bracket_the_attention_kernel():
    import ctypes
    from head_attention_forward_fa_amd import _native
    lib = _native.load()
    hip = ctypes.CDLL("libamdhip64.so.7")
    ev = [ctypes.c_void_p(), ctypes.c_void_p()]
    for e in ev:
        assert hip.hipEventCreate(ctypes.byref(e)) == 0
    inp = mi.make_inputs(dtype="bf16", seqlens=[700], num_heads=4, num_kv_heads=4,
                         head_dim_nope=128, v_dim=128, causal=True, seed=6)
    t = device_tensors(inp)
    torch.cuda.synchronize()
    _native.check(lib.mha_fwd_set_kernel_events(ev[0], ev[1]))
    try:
        run_gpu(inp, tensors=t)
    finally:
        _native.check(lib.mha_fwd_set_kernel_events(None, None))
    torch.cuda.synchronize()
    ms = ctypes.c_float()
    assert hip.hipEventElapsedTime(ctypes.byref(ms), ev[0], ev[1]) == 0
    assert 0.0 < ms.value < 1000.0
    for e in ev:
        hip.hipEventDestroy(e)


def test_all_sequences_empty_and_zero_max_seqlen():
    from head_attention_forward_fa_amd import mha_fwd
    dev = "cuda:0"
    q = torch.zeros(0, 2, 128, dtype=torch.bfloat16, device=dev)
    cu = torch.zeros(3, dtype=torch.int32, device=dev)
    o, lse = mha_fwd(q, q, q, cu_seqlens=cu, max_seqlen=0, causal=True)
    torch.cuda.synchronize()
    assert o.shape == (0, 2, 128) and lse.shape == (2, 0)


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_overflowing_lengths_are_refused_without_writes(dt):
    # max_seqlen 128 sizes the table for one tile per (sequence, head); a
    # 300-token sequence needs two, so the device refuses and writes nothing
    # (f32: a problem this small takes the direct item mapping, whose
    # workgroups check the lengths themselves)
    from head_attention_forward_fa_amd import mha_fwd
    inp = mi.make_inputs(dtype=dt, seqlens=[300], num_heads=2, num_kv_heads=2,
                         head_dim_nope=128, v_dim=128, causal=True, seed=5)
    t = device_tensors(inp)
    out = torch.full((300, 2, 128), 7.0,
                     dtype=torch.bfloat16 if dt == "bf16" else torch.float32, device="cuda:0")
    lse = torch.full((2, 300), 7.0, dtype=torch.float32, device="cuda:0")
    mha_fwd(t["q"], t["k"], t["v"], causal=True, cu_seqlens=t["cu_seqlens"], max_seqlen=128,
            out=out, lse=lse)
    torch.cuda.synchronize()
    assert bool((out == 7.0).all()) and bool((lse == 7.0).all())


# protocol 0: the next item reserved when an item starts, its entry read after
# a barrier (the float32 kernel);
# protocol 1: reserved and read in two steps near the end of an item, items
# with no key blocks included (the matrix-core kernel)
@pytest.mark.parametrize("protocol", [0, 1])
@pytest.mark.parametrize("block_m", [32, 256])
@pytest.mark.parametrize("grid", [0, 1, 7, 1000])
def test_scheduler_visits_every_item_once(block_m, grid, protocol):
    from head_attention_forward_fa_amd import mha_sched_visit
    rng = np.random.default_rng(block_m + grid)
    lens = rng.integers(0, 1500, size=23)
    lens[3] = 0
    lens[5] = 1
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    hq, hkv = 8, 2
    mx = int(lens.max())
    visits = mha_sched_visit(torch.from_numpy(cu).cuda(), mx, hq, hkv, True, block_m, grid,
                             protocol)
    torch.cuda.synchronize()
    tiles = (mx + block_m - 1) // block_m
    want = np.zeros((hq, len(lens), tiles), dtype=np.int32)
    for b, L in enumerate(lens):
        want[:, b, : (L + block_m - 1) // block_m] = 1
    assert np.array_equal(visits.cpu().numpy(), want)


@pytest.mark.parametrize("protocol", [0, 1])
@pytest.mark.parametrize("causal", [False, True])
def test_scheduler_many_groups_index_mode(causal, protocol):
    # more (sequence, KV head) groups than the prepass ranks in LDS: the
    # contiguous-range queue assignment must still cover every item once
    from head_attention_forward_fa_amd import mha_sched_visit
    rng = np.random.default_rng(9)
    lens = rng.integers(0, 600, size=700)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    hq, hkv = 8, 4
    mx = int(lens.max())
    visits = mha_sched_visit(torch.from_numpy(cu).cuda(), mx, hq, hkv, causal, 256, 0,
                             protocol)
    torch.cuda.synchronize()
    tiles = (mx + 255) // 256
    want = np.zeros((hq, len(lens), tiles), dtype=np.int32)
    for b, L in enumerate(lens):
        want[:, b, : (L + 255) // 256] = 1
    assert np.array_equal(visits.cpu().numpy(), want)


@pytest.mark.parametrize("protocol", [0, 1])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("nseq,hkv,maxlen", [(511, 4, 2600), (256, 8, 2600), (9, 1, 2600),
                                            (300, 2, 600)])
def test_scheduler_ranked_groups_cover_every_item_once(nseq, hkv, maxlen, causal, protocol):
    # groups ranked in LDS (up to 2048 of them, padded to a power of two for
    # the sort) and laid out chunk by chunk, round by round, in each queue
    # (short sequences: chunks of many groups)
    from head_attention_forward_fa_amd import mha_sched_visit
    rng = np.random.default_rng(nseq)
    lens = rng.integers(0, maxlen, size=nseq)
    lens[0] = 0
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    hq = 2 * hkv
    mx = int(lens.max())
    visits = mha_sched_visit(torch.from_numpy(cu).cuda(), mx, hq, hkv, causal, 256, 0,
                             protocol)
    torch.cuda.synchronize()
    tiles = (mx + 255) // 256
    want = np.zeros((hq, len(lens), tiles), dtype=np.int32)
    for b, L in enumerate(lens):
        want[:, b, : (L + 255) // 256] = 1
    assert np.array_equal(visits.cpu().numpy(), want)
