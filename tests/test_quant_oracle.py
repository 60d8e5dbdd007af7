"""Pins for the fp8 quantisation oracle (oracle/quantize.py).

* format facts: the table of finite E4M3 values (127 non-negative codes,
  largest 448 at 0x7E, smallest subnormal 2^-9 at 0x01, ascending);
* every finite code's own value rounds back to that code, signs included;
* exact midpoints between neighbouring values go to the even code, and the
  next float32 on either side goes to the nearer code;
* brute force: a pure-Python nearest-value search on random values;
* a library special case: torch's float32 -> float8_e4m3fn conversion on
  values inside the range, and the seeded input generator's quantiser;
* closed forms of the row quantiser: a zero row, the row maximum mapping to
  +-448, the scale being the float32 quotient amax / 448, and the error
  bound of round-to-nearest (half an E4M3 step);
* planted mistakes (ties away from zero, a wrong divisor) fail these pins.
"""

import math

import numpy as np
import pytest
import torch

from mha_inputs import to_e4m3_per_row
from oracle import quantize as oq
from oracle.attention import decode_e4m3


def test_table_facts():
    vals, codes = oq.e4m3_table()
    assert len(vals) == 127 and len(set(codes.tolist())) == 127
    assert np.all(np.diff(vals) > 0)
    assert vals[0] == 0.0 and codes[0] == 0x00
    assert vals[1] == 2.0 ** -9 and codes[1] == 0x01
    assert vals[-1] == 448.0 and codes[-1] == 0x7E
    assert vals[list(codes).index(0x38)] == 1.0


def test_every_code_rounds_to_itself():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    vals = decode_e4m3(codes).astype(np.float32)
    assert np.array_equal(oq.round_to_e4m3(vals), codes)


def test_midpoints_go_to_even_code():
    vals, codes = oq.e4m3_table()
    for i in range(len(vals) - 1):
        lo, hi = vals[i], vals[i + 1]
        mid = np.float32((lo + hi) / 2)
        assert float(mid) == (lo + hi) / 2            # exact in float32
        even = codes[i] if codes[i] % 2 == 0 else codes[i + 1]
        for sgn, sbit in ((1, 0), (-1, 0x80)):
            got = oq.round_to_e4m3(np.array([sgn * mid], dtype=np.float32))[0]
            assert got == (even | sbit), (lo, hi)
            up = np.nextafter(np.float32(sgn * mid), np.float32(sgn * 1e9))
            dn = np.nextafter(np.float32(sgn * mid), np.float32(0))
            assert oq.round_to_e4m3(np.array([up], dtype=np.float32))[0] == (codes[i + 1] | sbit)
            assert oq.round_to_e4m3(np.array([dn], dtype=np.float32))[0] == (codes[i] | sbit)


def _brute(y: float) -> int:
    best = None
    for c in range(0x7F):
        v = float(decode_e4m3(np.array([c], dtype=np.uint8))[0])
        d = abs(abs(y) - v)
        if best is None or d < best[0] or (d == best[0] and c % 2 == 0):
            best = (d, c)
    return best[1] | (0x80 if math.copysign(1.0, y) < 0 else 0)


def test_matches_brute_force_search():
    rng = np.random.default_rng(3)
    y = np.concatenate([rng.uniform(-448, 448, 300), rng.uniform(-0.02, 0.02, 200),
                        rng.standard_normal(200) * 4]).astype(np.float32)
    got = oq.round_to_e4m3(y)
    assert [int(c) for c in got] == [_brute(float(v)) for v in y]


def test_matches_torch_conversion_in_range():
    rng = np.random.default_rng(4)
    y = np.concatenate([rng.uniform(-448, 448, 20000),
                        rng.standard_normal(20000) * 2.0 ** rng.integers(-12, 8, 20000)])
    y = np.clip(y, -448, 448).astype(np.float32)
    ref = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(oq.round_to_e4m3(y), ref)


def test_row_quantiser_matches_input_generator():
    rng = np.random.default_rng(5)
    x = (rng.standard_normal((50, 4, 128)) * rng.lognormal(0, 1, (50, 4, 1))).astype(np.float32)
    codes, scales = oq.quantize_rows(x)
    gcodes, gscales = to_e4m3_per_row(x)
    assert np.array_equal(scales, gscales)
    assert np.array_equal(codes, gcodes)


def test_row_closed_forms():
    rng = np.random.default_rng(6)
    x = rng.standard_normal((8, 64)).astype(np.float32)
    x[3] = 0.0
    codes, scales = oq.quantize_rows(x)
    assert scales[3] == 1.0 and np.all(codes[3] == 0)
    for r in (0, 1, 2, 4, 5, 6, 7):
        amax = np.abs(x[r]).max()
        assert scales[r] == np.float32(amax / np.float32(448.0))
        j = int(np.argmax(np.abs(x[r])))
        assert codes[r, j] == (0x7E if x[r, j] > 0 else 0xFE)
        # round to nearest: at most half a step of the E4M3 grid at that magnitude
        deq = decode_e4m3(codes[r]) * float(scales[r])
        y = np.abs(x[r].astype(np.float64)) / float(scales[r])
        step = np.where(y >= 2.0 ** -6, 2.0 ** (np.floor(np.log2(np.maximum(y, 2.0 ** -6))) - 3), 2.0 ** -9)
        assert np.all(np.abs(deq - x[r]) <= 0.5 * step * float(scales[r]) * (1 + 1e-6) + 1e-30)


def test_bf16_rows_use_exact_values():
    x = np.array([[1.0, -3.0, 0.5, 0.0] * 16], dtype=np.float32)
    bits = (x.view(np.uint32) >> 16).astype(np.uint16)
    c1, s1 = oq.quantize_bf16_rows(bits)
    c2, s2 = oq.quantize_rows(x)
    assert np.array_equal(c1, c2) and np.array_equal(s1, s2)
    assert s1[0] == np.float32(3.0 / 448.0)


@pytest.mark.parametrize("mutant", ["ties_away", "divisor"])
def test_planted_mistakes_fail_pins(mutant, monkeypatch):
    if mutant == "ties_away":
        def bad(y):
            vals, codes = oq.e4m3_table()
            a = np.abs(np.asarray(y, dtype=np.float64)).ravel()
            hi = np.clip(np.searchsorted(vals, a), 0, len(vals) - 1)
            lo = np.clip(hi - 1, 0, len(vals) - 1)
            mag = np.where(vals[hi] - a <= a - vals[lo], codes[hi], codes[lo]).astype(np.uint8)
            return (mag | (np.signbit(np.asarray(y).ravel()).astype(np.uint8) << 7)).reshape(np.shape(y))
        monkeypatch.setattr(oq, "round_to_e4m3", bad)
        with pytest.raises(AssertionError):
            test_midpoints_go_to_even_code()
    else:
        monkeypatch.setattr(oq, "E4M3_MAX", 447.0)
        with pytest.raises(AssertionError):
            test_row_closed_forms()
