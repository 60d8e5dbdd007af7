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
