"""mha_fwd's own key splits (few, long work items): the HIP path against the
float64 oracle, and the merge writes nothing past the real token count
(the partials are laid out for batch x max_seqlen tokens)."""

import numpy as np
import pytest
import torch

import mha_inputs as mi
from _util import TOL_LSE, TOL_O, device_tensors, max_abs, oracle_full, to_f64

pytestmark = pytest.mark.gpu

CASES = [
    # dtype, lengths, Hq, Hkv, Dn, Dr, Dv, causal
    ("bf16", [2048], 2, 2, 128, 0, 128, True),
    ("bf16", [2048, 700, 1500], 2, 1, 128, 0, 128, True),
    ("bf16", [1800, 0, 1100], 4, 2, 128, 0, 128, False),
    ("bf16", [1500], 2, 2, 128, 64, 128, True),
    ("bf16", [1300, 200], 2, 2, 64, 0, 64, True),
    ("fp8", [2048, 333], 2, 2, 128, 0, 128, True),
    ("fp8", [1400], 2, 1, 128, 64, 128, True),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}-{c[1]}-{c[2]}x{c[3]}-{c[4]}+{c[5]}-{'c' if c[7] else 'nc'}")
def test_auto_split_matches_oracle_and_stays_in_bounds(case):
    from head_attention_forward_fa_amd import mha_fwd, mha_fwd_auto_splits
    dt, lens, hq, hkv, dn, dr, dv, causal = case
    inp = mi.make_inputs(dtype=dt, seqlens=lens, num_heads=hq, num_kv_heads=hkv,
                         head_dim_nope=dn, head_dim_rope=dr, v_dim=dv, causal=causal,
                         seed=11, name=str(case))
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    splits = mha_fwd_auto_splits(len(lens), inp.max_seqlen, hq, causal, dv, cus)
    print("case", case, "splits", splits, flush=True)
    assert splits > 1, "the case is meant to take the split path"
    t = device_tensors(inp)
    T = inp.total_tokens
    odt = torch.bfloat16
    guard = 97
    o_buf = torch.full((T + guard, hq, dv), 3.0, dtype=odt, device="cuda:0")
    l_buf = torch.full((hq * T + guard,), 5.0, dtype=torch.float32, device="cuda:0")
    o, lse = o_buf[:T], l_buf[:hq * T].view(hq, T)
    mha_fwd(t["q"], t["k"], t["v"], causal=causal, cu_seqlens=t["cu_seqlens"],
            max_seqlen=inp.max_seqlen, q_rope=t["q_rope"], k_rope=t["k_rope"],
            q_scale=t["q_scale"], k_scale=t["k_scale"], softmax_scale=inp.softmax_scale,
            out=o, lse=lse)
    torch.cuda.synchronize()
    assert bool((o_buf[T:] == 3.0).all()), "O written past the last token"
    assert bool((l_buf[hq * T:] == 5.0).all()), "LSE written past its end"
    ref_o, ref_lse = oracle_full(inp)
    o64, l64 = to_f64(o), to_f64(lse)
    assert np.all(np.isfinite(o64))
    eo, el = max_abs(o64, ref_o), max_abs(l64, ref_lse)
    assert eo <= TOL_O[dt], f"O max-abs {eo}"
    assert el <= TOL_LSE, f"LSE max-abs {el}"


@pytest.mark.parametrize("num_splits", [1, 3])  # 1: mha_fwd's own splits; 3: mha_fwd_splitkv
def test_split_paths_refuse_lengths_above_max_seqlen_without_writes(num_splits):
    """A length above max_seqlen makes the prepass refuse (the partials are
    laid out for batch x max_seqlen tokens): no work item runs and the merge
    writes nothing, so O and LSE keep what they held."""
    from head_attention_forward_fa_amd import mha_fwd, mha_fwd_auto_splits
    inp = mi.make_inputs(dtype="bf16", seqlens=[2048, 600], num_heads=2, num_kv_heads=2,
                         head_dim_nope=128, v_dim=128, causal=True, seed=12)
    short = 2000  # the first sequence is longer
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    if num_splits == 1:
        assert mha_fwd_auto_splits(2, short, 2, True, 128, cus) > 1, "meant to split by itself"
    t = device_tensors(inp)
    T = inp.total_tokens
    o = torch.full((T, 2, 128), 7.0, dtype=torch.bfloat16, device="cuda:0")
    lse = torch.full((2, T), 7.0, dtype=torch.float32, device="cuda:0")
    mha_fwd(t["q"], t["k"], t["v"], causal=True, cu_seqlens=t["cu_seqlens"], max_seqlen=short,
            num_splits=num_splits, out=o, lse=lse)
    torch.cuda.synchronize()
    assert bool((o == 7.0).all()) and bool((lse == 7.0).all())
