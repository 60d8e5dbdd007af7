"""mha_fwd_noalloc (the entry point that allocates nothing on the device)
against mha_fwd, through the C ABI: two calls in a row on the library's fixed
workspace, the second with a smaller problem (it reuses the state the first
left), each equal to mha_fwd's output bit for bit (same kernels; neither
call's shape makes mha_fwd split keys by itself); float32, bf16 and fp8;
and a work table beyond the fixed workspace refused before any launch."""

import pytest
import torch

import mha_inputs as mi
from _util import device_tensors, run_gpu

pytestmark = pytest.mark.gpu


def _noalloc(inp, t):
    from head_attention_forward_fa_amd import mha_fwd_noalloc
    vdt = torch.float32 if inp.dtype == "f32" else torch.bfloat16
    o = torch.full((inp.total_tokens, inp.num_heads, inp.v_dim), 9.0, dtype=vdt, device="cuda:0")
    lse = torch.full((inp.num_heads, inp.total_tokens), 9.0, dtype=torch.float32,
                     device="cuda:0")
    mha_fwd_noalloc(t["q"], t["k"], t["v"], out=o, lse=lse, cu_seqlens=t["cu_seqlens"],
                    max_seqlen=inp.max_seqlen, causal=inp.causal, q_rope=t["q_rope"],
                    k_rope=t["k_rope"], q_scale=t["q_scale"], k_scale=t["k_scale"],
                    softmax_scale=inp.softmax_scale)
    torch.cuda.synchronize()
    return o, lse


PAIRS = [
    # (first call, second smaller call): dtype, lengths, Hq, Hkv, Dn, Dr, Dv, causal
    (("bf16", [1100, 300, 517], 32, 8, 128, 0, 128, True),
     ("bf16", [200, 77], 4, 4, 128, 0, 128, True)),
    (("fp8", [900, 41], 4, 2, 128, 0, 128, True),
     ("fp8", [130], 2, 2, 128, 0, 128, False)),
    (("bf16", [700, 650], 4, 4, 128, 64, 128, False),
     ("f32", [100, 3], 2, 2, 64, 0, 64, True)),
]


@pytest.mark.parametrize("pair", PAIRS, ids=lambda p: f"{p[0][0]}-then-{p[1][0]}")
def test_noalloc_equals_mha_fwd_on_two_calls(pair):
    from head_attention_forward_fa_amd import mha_fwd_auto_splits
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    for seed, case in enumerate(pair):
        dt, lens, hq, hkv, dn, dr, dv, causal = case
        inp = mi.make_inputs(dtype=dt, seqlens=lens, num_heads=hq, num_kv_heads=hkv,
                             head_dim_nope=dn, head_dim_rope=dr, v_dim=dv, causal=causal,
                             seed=21 + seed, name=str(case))
        if dt != "f32":
            assert mha_fwd_auto_splits(len(lens), inp.max_seqlen, hq, causal, dv, cus) == 1
        print("case", case, flush=True)
        t = device_tensors(inp)
        o_ref, l_ref = run_gpu(inp, tensors=t)
        o, lse = _noalloc(inp, t)
        assert torch.equal(o, o_ref) and torch.equal(lse, l_ref), case


def test_noalloc_refuses_a_table_beyond_its_workspace():
    import ctypes
    from head_attention_forward_fa_amd import _native as nat
    lib = nat.load()
    fake = 0x1000  # never dereferenced: the size check comes before any launch
    # 64 sequences x 64 heads x 256 query tiles = 2^20 work items, 16 MiB of table
    st = lib.mha_fwd_noalloc(fake, fake, fake, fake, fake, fake, 64, 65536, 64, 64, 128, 0, 128,
                             None, None, 1, 0.0, nat.MHA_DTYPE_BF16, None, None, None)
    assert st == nat.MHA_ERR_INVALID_ARG
    msg = lib.mha_fwd_last_error().decode()
    assert "mha_fwd_noalloc" in msg and "16777216" in msg, msg
    del ctypes
