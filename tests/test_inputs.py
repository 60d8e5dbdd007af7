"""The seeded generators: deterministic, with the stated shapes and ranges."""

import numpy as np

import mha_inputs as mi


def test_same_seed_same_bits():
    a = mi.make_inputs(dtype="bf16", seqlens=[5, 9], num_heads=4, num_kv_heads=2,
                       head_dim_nope=8, head_dim_rope=4, v_dim=8, causal=True, seed=3)
    b = mi.make_inputs(dtype="bf16", seqlens=[5, 9], num_heads=4, num_kv_heads=2,
                       head_dim_nope=8, head_dim_rope=4, v_dim=8, causal=True, seed=3)
    for f in ("q", "k", "v", "q_rope", "k_rope", "cu_seqlens"):
        assert np.array_equal(getattr(a, f), getattr(b, f))
    c = mi.make_inputs(dtype="bf16", seqlens=[5, 9], num_heads=4, num_kv_heads=2,
                       head_dim_nope=8, head_dim_rope=4, v_dim=8, causal=True, seed=4)
    assert not np.array_equal(a.q, c.q)


def test_shapes_and_dtypes():
    x = mi.make_inputs(dtype="fp8", seqlens=[3, 0, 4], num_heads=4, num_kv_heads=1,
                       head_dim_nope=16, v_dim=8, causal=True, seed=0)
    assert x.q.dtype == np.uint8 and x.q.shape == (7, 4, 16)
    assert x.k.dtype == np.uint8 and x.k.shape == (7, 1, 16)
    assert x.v.dtype == np.uint16 and x.v.shape == (7, 1, 8)
    assert x.q_scale.shape == (7, 4) and np.all(x.q_scale > 0)
    assert x.k_scale.shape == (7, 1) and np.all(x.k_scale > 0)
    assert list(x.cu_seqlens) == [0, 3, 3, 7] and x.cu_seqlens.dtype == np.int32
    # per-row amax quantises to the largest E4M3 magnitude (code 0x7E)
    assert np.all((x.q & 0x7F).max(axis=-1) == 0x7E)


def test_ragged_workload_lengths():
    rng = np.random.default_rng(0)
    lens = mi.ragged_lengths(rng)
    assert len(lens) == 16 and lens.min() >= 64 and lens.max() <= 8192
    spec = mi.WORKLOADS["bf16_varlen_gqa_causal_16seq_hq32_hkv8_d128"]
    assert spec["num_heads"] == 32 and spec["num_kv_heads"] == 8


def test_bf16_encoding_rounds_to_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5], dtype=np.float32)
    bits = mi.to_bf16_bits(x)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: even mantissa (1.0) wins;
    # 1 + 3*2^-8 is a tie between 1 + 2^-7 and 1 + 2^-6: even (1 + 2^-6) wins.
    assert list(bits) == [0x3F80, 0x3F80, 0x3F82, 0xC020]


def test_flop_count_matches_metric():
    x = mi.make_inputs(dtype="bf16", seqlens=[4096] * 4, num_heads=1, num_kv_heads=1,
                       head_dim_nope=2, v_dim=2, causal=True, seed=0)
    assert mi.attention_flops(x) == 4 * 4 * 1 * 4096 * 4096 * 2 / 2
