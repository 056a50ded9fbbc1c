"""Pins of the oracle's FP4 / FP8 / E8M0 codecs against sources other than the oracle.

* hand-typed OCP tables (tests/golden/*.txt, each citing its specification section),
* torch's own float8_e4m3fn conversion (a library implementation of the same format),
* round-trip and tie-case properties that follow from round-to-nearest-even.
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _rows(name):
    out = []
    with open(os.path.join(GOLD, name)) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                a, b = line.split()
                out.append((a, b))
    return out


def _same(a, b):
    if math.isnan(b):
        return math.isnan(a)
    return a == b and math.copysign(1, a) == math.copysign(1, b)


def test_e2m1_table_matches_ocp():
    rows = _rows("e2m1_values.txt")
    assert len(rows) == 16
    for code, val in rows:
        assert _same(oracle.fp4_value(int(code, 16)), float(val)), code


def test_e4m3fn_all_codes_match_torch():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    for c in range(256):
        assert _same(oracle.fp8_value(c), float(ref[c])), hex(c)


def test_e4m3fn_spot_values_match_ocp():
    for code, val in _rows("e4m3fn_spot.txt"):
        assert _same(oracle.fp8_value(int(code, 16)), float(val)), code


def test_e8m0_spot_values_match_ocp():
    for code, val in _rows("e8m0_spot.txt"):
        v = oracle.e8m0_value(int(code))
        if val == "nan":
            assert math.isnan(v)
        else:
            assert v == float(val), code
    for c in range(255):
        assert oracle.e8m0_value(c) == math.ldexp(1.0, c - 127)


def _group(vals, pad=0.0):
    g = np.full((1, 32), pad, np.float32)
    g[0, :len(vals)] = vals
    return g


def test_fp4_rounding_table():
    # one group per test value; an element of 7.5 pins the shared exponent at 0
    for mag, code in _rows("e2m1_rounding.txt"):
        for sign in (1.0, -1.0):
            g = _group([7.5, sign * float(mag)])
            codes, scales = oracle.quantize_mxfp4(g)
            assert scales[0, 0] == 127
            c = int(codes[0, 0] >> 4)  # element 1 lives in the high nibble of byte 0
            assert c & 7 == int(code), (mag, sign)
            assert (c >> 3) == (1 if sign < 0 else 0), (mag, sign)


def test_fp4_scale_rule():
    # amax in [2^(k+2), 2^(k+3)) -> e = k  (floor(log2 amax) - 2)
    for k in range(-20, 21):
        for amax in (2.0 ** (k + 2), 1.5 * 2.0 ** (k + 2), 
                     np.nextafter(np.float32(2.0 ** (k + 3)), np.float32(0))):
            g = _group([np.float32(amax)])
            _, s = oracle.quantize_mxfp4(g)
            assert int(s[0, 0]) - 127 == k, (k, amax)
    # zero group -> scale code 0, all codes +0
    c, s = oracle.quantize_mxfp4(np.zeros((1, 32), np.float32))
    assert s[0, 0] == 0 and not c.any()
    # tiny amax clamps at -127
    g = _group([np.float32(1e-44)])
    _, s = oracle.quantize_mxfp4(g)
    assert s[0, 0] == 0


def test_fp4_round_trip_every_code_and_scale():
    vals = [oracle.fp4_value(c) for c in range(16)]
    for e in (-30, -3, -1, 0, 1, 7, 40):
        # element 0 = 6 * 2^e fixes the exponent; elements 1..15 carry every other code
        x = np.array([6.0 * 2.0 ** e] + [v * 2.0 ** e for v in vals[:15]] + [0.0] * 16,
                     np.float32)
        codes, scales = oracle.quantize_mxfp4(x[None])
        assert int(scales[0, 0]) - 127 == e
        got = [(int(codes[0, i // 2]) >> (4 * (i % 2))) & 15 for i in range(16)]
        assert got == [7] + list(range(15)), e
        back = oracle.dequant_mxfp4(codes, scales)[0]
        assert np.array_equal(back, x.astype(np.float64))


def test_fp4_nibble_order():
    # element 2i -> low nibble, 2i+1 -> high nibble
    x = np.zeros((1, 32), np.float32)
    x[0, 0], x[0, 1], x[0, 31] = 1.0, 6.0, -0.5
    codes, scales = oracle.quantize_mxfp4(x)
    assert scales[0, 0] == 127
    assert codes[0, 0] == (0x7 << 4) | 0x2
    assert codes[0, 15] == (0x9 << 4)


def test_fp8_matches_torch_rounding():
    # With the exponent pinned (an element of 448 * 2^e), every other element's code must
    # equal torch's float -> float8_e4m3fn conversion of x / 2^e (RNE, in range).
    rng = np.random.default_rng(7)
    for e in (-10, -2, 0, 3):
        for _ in range(40):
            mags = np.concatenate([rng.uniform(0, 448, 15), 2.0 ** rng.uniform(-12, 8.8, 16)])
            signs = rng.choice([-1.0, 1.0], 31)
            v = (mags * signs).astype(np.float32)
            x = np.concatenate([[448.0], v]).astype(np.float32) * np.float32(2.0 ** e)
            codes, scales = oracle.quantize_mxfp8(x[None])
            assert int(scales[0, 0]) - 127 == e
            ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
            assert np.array_equal(codes[0, 1:], ref)


def test_fp8_ties_and_saturation():
    # exponent pinned at 0 by an element in [256, 512)
    # 464 lies between 448 and the (absent) 480 -> saturates to 448 (0x7E)
    x = _group([300.0, 464.0, 511.0, -500.0, 0.5 * 2 ** -9, 1.5 * 2 ** -9, 2.5 * 2 ** -9])
    codes, scales = oracle.quantize_mxfp8(x)
    assert scales[0, 0] == 127 + 0
    assert list(codes[0, 1:7]) == [0x7E, 0x7E, 0xFE, 0x00, 0x02, 0x02]


def test_fp8_round_trip_all_codes():
    vals = [oracle.fp8_value(c) for c in range(0x7F)]
    for e in (-5, 0, 9):
        for start in range(0, 127, 31):
            chunk = vals[start:start + 31]
            x = np.array([448.0] + chunk + [0.0] * (31 - len(chunk)), np.float64) * 2.0 ** e
            codes, scales = oracle.quantize_mxfp8(x.astype(np.float32)[None])
            assert int(scales[0, 0]) - 127 == e
            assert list(codes[0, 1:1 + len(chunk)]) == list(range(start, start + len(chunk)))


def test_dequant_is_code_times_scale():
    rng = np.random.default_rng(3)
    codes = rng.integers(0, 256, (5, 64), dtype=np.uint8)
    scales = rng.integers(100, 150, (5, 4), dtype=np.uint8)
    out = oracle.dequant_mxfp4(codes, scales)
    tab = np.array([float(v) for _, v in _rows("e2m1_values.txt")])
    for r in range(5):
        for i in range(128):
            c = (int(codes[r, i // 2]) >> (4 * (i % 2))) & 15
            assert out[r, i] == tab[c] * 2.0 ** (int(scales[r, i // 32]) - 127)


@pytest.mark.parametrize("seed", [0, 1])
def test_quantizers_accept_normal_data(seed):
    x = np.random.default_rng(seed).standard_normal((64, 512)).astype(np.float32)
    c4, s4 = oracle.quantize_mxfp4(x)
    d4 = oracle.dequant_mxfp4(c4, s4)
    # error bound: half the widest grid gap (4 -> 6) below 6, and 8 - 6 for the saturated
    # range (6, 8), both in units of the group's scale 2^e
    step = 2.0 ** (s4.astype(np.float64) - 127).repeat(32, axis=1)
    assert np.all(np.abs(d4 - x) <= np.where(np.abs(x) > 6 * step, 2.0, 1.0) * step)
    c8, s8 = oracle.quantize_mxfp8(x)
    d8 = oracle.dequant_mxfp8(c8, s8)
    # E4M3: half an ulp (2^-4 relative) in range, 2^(e-10) in the subnormal range, and
    # up to 512 - 448 = 64 units of 2^e for the saturated range (448, 512)
    sc8 = 2.0 ** (s8.astype(np.float64) - 127).repeat(32, axis=1)
    bound = np.where(np.abs(x) > 448 * sc8, 64 * sc8,
                     np.maximum(np.abs(x) * 2.0 ** -4, sc8 * 2.0 ** -10))
    assert np.all(np.abs(d8 - x) <= bound)
