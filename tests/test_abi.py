"""The C ABI on the CPU: the library loads, exports what include/mha_fwd.h
declares, and rejects malformed arguments before any HIP call."""

import math
import os
import re

import pytest

from head_attention_forward_fa_amd import _native as nat

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x1000  # never dereferenced: every call below fails validation first


def declared_functions():
    names = set()
    inc = os.path.join(ROOT, "include")
    for f in os.listdir(inc):
        if f.endswith(".h"):
            text = open(os.path.join(inc, f)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names.update(re.findall(r"^[A-Za-z_][\w\s\*]*?\b(mha_\w+)\s*\(", text, flags=re.M))
    return sorted(names)


def test_library_exports_every_declared_function():
    lib = nat.load()
    names = declared_functions()
    assert set(names) >= {"mha_fwd", "mha_fwd_last_error", "mha_fwd_supported", "mha_sched_visit"}
    for n in names:
        assert hasattr(lib, n), n
    assert set(nat.EXPORTS) == set(names)


def call(**over):
    args = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, cu=FAKE, batch=1, max_seqlen=16,
                hq=4, hkv=2, dn=128, dr=0, dv=128, q_rope=None, k_rope=None, causal=1,
                scale=0.0, dtype=nat.MHA_DTYPE_BF16, q_scale=None, k_scale=None, stream=None)
    args.update(over)
    lib = nat.load()
    return lib.mha_fwd(args["q"], args["k"], args["v"], args["o"], args["lse"], args["cu"],
                       args["batch"], args["max_seqlen"], args["hq"], args["hkv"], args["dn"],
                       args["dr"], args["dv"], args["q_rope"], args["k_rope"], args["causal"],
                       args["scale"], args["dtype"], args["q_scale"], args["k_scale"],
                       args["stream"])


BAD = [
    dict(q=None), dict(lse=None), dict(cu=None),
    dict(batch=0), dict(max_seqlen=-1), dict(hq=0), dict(hkv=3), dict(hq=4096, hkv=1),
    dict(dn=0), dict(dr=-1), dict(dv=0),
    dict(dr=64),                                  # rope depth without rope pointers
    dict(q_rope=FAKE, k_rope=FAKE),               # rope pointers without depth
    dict(dr=64, q_rope=FAKE),                     # only one rope pointer
    dict(causal=2), dict(dtype=7),
    dict(dtype=nat.MHA_DTYPE_FP8_E4M3),           # fp8 without scales
    dict(dtype=nat.MHA_DTYPE_FP8_E4M3, q_scale=FAKE),
    dict(dtype=nat.MHA_DTYPE_FP8_E4M3_FASTACC),   # fast-accumulation fp8 without scales
    dict(dtype=nat.MHA_DTYPE_FP8_E4M3_FASTACC, k_scale=FAKE),
    dict(q_scale=FAKE, k_scale=FAKE),             # scales with bf16
    dict(scale=math.nan), dict(scale=math.inf),
    # alignment: 16 bytes for the tensors moved in 16-byte units, 4 for the rest
    dict(q=FAKE + 2), dict(k=FAKE + 8), dict(v=FAKE + 4), dict(o=FAKE + 2),
    dict(dr=64, q_rope=FAKE + 8, k_rope=FAKE), dict(dr=64, q_rope=FAKE, k_rope=FAKE + 2),
    dict(lse=FAKE + 2), dict(cu=FAKE + 1),
    dict(dtype=nat.MHA_DTYPE_FP8_E4M3, q_scale=FAKE + 2, k_scale=FAKE),
    dict(dtype=nat.MHA_DTYPE_FP8_E4M3, q_scale=FAKE, k_scale=FAKE + 1),
]


@pytest.mark.parametrize("over", BAD)
def test_invalid_arguments_rejected(over):
    assert call(**over) == nat.MHA_ERR_INVALID_ARG
    assert nat.load().mha_fwd_last_error().decode()


@pytest.mark.parametrize("over", [dict(dn=96, dv=96), dict(dv=64),
                                  dict(dtype=nat.MHA_DTYPE_FP8_E4M3, q_scale=FAKE,
                                       k_scale=FAKE, dn=64, dv=64),
                                  dict(dtype=nat.MHA_DTYPE_FP8_E4M3, q_scale=FAKE,
                                       k_scale=FAKE, dr=32, q_rope=FAKE, k_rope=FAKE)])
def test_unsupported_shapes(over):
    assert call(**over) == nat.MHA_ERR_UNSUPPORTED


def test_zero_max_seqlen_is_a_no_op():
    assert call(max_seqlen=0) == nat.MHA_OK
    assert nat.load().mha_fwd_last_error().decode() == ""


def test_supported_set():
    lib = nat.load()
    want = {
        nat.MHA_DTYPE_F32: {(64, 0, 64), (128, 0, 128), (128, 64, 128)},
        nat.MHA_DTYPE_BF16: {(64, 0, 64), (128, 0, 128), (128, 64, 128)},
        nat.MHA_DTYPE_FP8_E4M3: {(128, 0, 128), (128, 64, 128)},
        nat.MHA_DTYPE_FP8_E4M3_FASTACC: {(128, 0, 128), (128, 64, 128)},
    }
    for dt, shapes in want.items():
        for dn in (32, 64, 96, 128, 192, 256):
            for dr in (0, 32, 64):
                for dv in (64, 128):
                    assert bool(lib.mha_fwd_supported(dt, dn, dr, dv)) == ((dn, dr, dv) in shapes)


def test_sched_visit_validation():
    lib = nat.load()
    for bad_block_m in (64, 128):
        assert lib.mha_sched_visit(FAKE, 1, 16, 4, 2, 1, bad_block_m, 0, 1, FAKE,
                                   None) == nat.MHA_ERR_INVALID_ARG
    assert lib.mha_sched_visit(FAKE, 1, 16, 4, 2, 1, 256, 0, 1, None, None) == nat.MHA_ERR_INVALID_ARG
    assert lib.mha_sched_visit(FAKE, 1, 16, 4, 2, 1, 256, -1, 1, FAKE, None) == nat.MHA_ERR_INVALID_ARG
    for bad_protocol in (-1, 2):
        assert lib.mha_sched_visit(FAKE, 1, 16, 4, 2, 1, 256, 0, bad_protocol, FAKE,
                                   None) == nat.MHA_ERR_INVALID_ARG
    assert lib.mha_sched_visit(FAKE, 1, 0, 4, 2, 1, 256, 0, 1, FAKE, None) == nat.MHA_OK


def test_set_kernel_events_validation():
    lib = nat.load()
    assert lib.mha_fwd_set_kernel_events(FAKE, None) == nat.MHA_ERR_INVALID_ARG
    assert lib.mha_fwd_set_kernel_events(None, FAKE) == nat.MHA_ERR_INVALID_ARG
    assert lib.mha_fwd_set_kernel_events(None, None) == nat.MHA_OK


def test_python_binding_fast_accum_needs_fp8():
    import torch
    from head_attention_forward_fa_amd import mha_fwd
    q = torch.zeros(2, 1, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        mha_fwd(q, q, q, cu_seqlens=torch.tensor([0, 2], dtype=torch.int32), max_seqlen=2,
                fp8_fast_accum=True)


def test_python_binding_rejects_cpu_tensors():
    import torch
    from head_attention_forward_fa_amd import mha_fwd
    q = torch.zeros(2, 1, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        mha_fwd(q, q, q, cu_seqlens=torch.tensor([0, 2], dtype=torch.int32), max_seqlen=2)


QBAD = [
    dict(dtype=nat.MHA_DTYPE_FP8_E4M3), dict(dtype=9),
    dict(rows=-1), dict(rows=1 << 31), dict(cols=0), dict(cols=4), dict(cols=12),
    dict(cols=520), dict(x=None), dict(codes=None), dict(scales=None),
    dict(x=FAKE + 8), dict(codes=FAKE + 4), dict(scales=FAKE + 2),
]


@pytest.mark.parametrize("over", QBAD)
def test_quantize_fp8_validation(over):
    a = dict(x=FAKE, dtype=nat.MHA_DTYPE_BF16, rows=16, cols=128, codes=FAKE, scales=FAKE)
    a.update(over)
    lib = nat.load()
    st = lib.mha_quantize_fp8(a["x"], a["dtype"], a["rows"], a["cols"], a["codes"], a["scales"],
                              None)
    assert st == nat.MHA_ERR_INVALID_ARG
    assert lib.mha_fwd_last_error()


def test_quantize_fp8_zero_rows_is_a_no_op():
    lib = nat.load()
    assert lib.mha_quantize_fp8(None, nat.MHA_DTYPE_F32, 0, 64, None, None, None) == nat.MHA_OK


def test_auto_splits_rule():
    from head_attention_forward_fa_amd import mha_fwd_auto_splits as auto
    cus = 256
    assert auto(4, 4096, 32, True, 128, cus) == 1        # many items: no split
    assert auto(2, 8192, 16, True, 128, cus) == 1
    assert auto(1, 16384, 4, False, 128, cus) == 1       # one full-length item per CU
    # one causal sequence, 4 heads: 256 items, the longest 256 blocks against
    # 130 blocks of work per CU: ceil(1.2 x 256 / 130) splits
    assert auto(1, 16384, 4, True, 128, cus) == 3
    assert auto(1, 16384, 2, True, 128, cus) == 5         # 65 blocks per CU
    assert auto(1, 2048, 2, True, 128, cus) == 4         # capped at 8 blocks per split
    assert auto(1, 960, 2, True, 128, cus) == 1          # fewer than 16 key blocks
    assert auto(1, 1024, 2, True, 128, cus) == 2
    assert auto(1, 1 << 20, 1, True, 128, 4096) <= 8     # capped at 8 splits
    # 1 GiB of float32 partials at most: 2 x 2^20 tokens x 64 heads x 128 x 4 B > 1 GiB
    assert auto(2, 1 << 20, 64, False, 128, 1 << 20) == 1
    for bad in [(0, 100, 1), (1, 0, 1), (1, 100, 0)]:
        assert auto(*bad, True, 128, cus) == 1
    assert auto(1, 2048, 2, True, 128, 0) == 1
