"""Host-side pieces of bench.py: the peak each dtype path is rated against."""

import types

import pytest

import bench


def _inp(dtype, dn=128, dr=0, dv=128):
    return types.SimpleNamespace(dtype=dtype, head_dim_nope=dn, head_dim_rope=dr, v_dim=dv)


def test_bf16_and_fp32_peaks():
    assert bench.peak_for(_inp("bf16")) == pytest.approx(2500.0)
    assert bench.peak_for(_inp("f32")) == pytest.approx(157.3)


def test_exact_fp8_is_rated_at_the_bf16_rate():
    # the default fp8 path decodes the codes to bf16: every product at the bf16 rate
    assert bench.peak_for(_inp("fp8")) == pytest.approx(2500.0)
    assert bench.peak_for(_inp("fp8", dr=64)) == pytest.approx(2500.0)


def test_fast_fp8_is_rated_at_the_time_weighted_blend():
    # nope Q K^T at the fp8 rate (5000), P V and a rope Q K^T at the bf16 rate
    assert bench.peak_for(_inp("fp8"), fast_accum=True) == pytest.approx(
        256 / (128 / 5000 + 128 / 2500))
    assert bench.peak_for(_inp("fp8", dr=64), fast_accum=True) == pytest.approx(
        320 / (128 / 5000 + 192 / 2500))


def test_profiled_kernel_follows_the_dtype():
    assert bench.kernel_of("f32") == "attn_fwd_f32_kernel"
    for dt in ("bf16", "fp8"):
        assert bench.kernel_of(dt) == "attn_fwd_mfma_kernel"
    # a profile summary is keyed by kernel and workload, and its source hash
    # covers that kernel's own sources
    assert bench.profile_path("w", "attn_fwd_f32_kernel").endswith("attn_fwd_f32_kernel_w.md")
    assert bench.kernel_sources_sha256("attn_fwd_f32_kernel") != bench.kernel_sources_sha256(
        "attn_fwd_mfma_kernel")


def test_cpu_model_names_the_host():
    s = bench.cpu_model()
    assert "logical CPUs" in s and len(s) > 20
