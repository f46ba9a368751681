"""Pins of the oracle's scalar conversions (E4M3 decode, BF16 decode, BF16 rounding).

Each test ties the oracle to something other than its own formula: the OCP
FP8 specification's values (hand-derived golden file), torch's independent
float8_e4m3fn / bfloat16 conversions, or exact rational arithmetic.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_e4m3():
    rows = []
    with open(os.path.join(GOLDEN, "e4m3_special_values.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            code, val = line.split()[:2]
            rows.append((int(code, 16), val))
    return rows


def test_e4m3_golden_special_values():
    rows = _golden_e4m3()
    assert len(rows) >= 20
    got = oracle.e4m3_value(np.array([c for c, _ in rows], np.uint8))
    for (code, val), g in zip(rows, got):
        if val == "nan":
            assert math.isnan(g), hex(code)
        elif val == "-0":
            assert g == 0.0 and math.copysign(1.0, g) < 0, hex(code)
        else:
            assert Fraction(g) == Fraction(val), (hex(code), g, val)
            if Fraction(val) == 0:
                assert math.copysign(1.0, g) > 0


def test_e4m3_matches_torch_on_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    mine = oracle.e4m3_value(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(mine), nan)
    assert set(np.nonzero(nan)[0].tolist()) == {0x7F, 0xFF}
    assert np.array_equal(mine[~nan], ref[~nan])
    assert np.array_equal(np.signbit(mine[~nan]), np.signbit(ref[~nan]))
    assert (~nan).sum() == 254


def test_e4m3_structure():
    v = oracle.e4m3_value(np.arange(256, dtype=np.uint8))
    pos = v[:0x7F]
    assert np.all(np.diff(pos) > 0), "codes 0x00..0x7E must increase strictly"
    assert pos[-1] == 448.0
    neg = v[0x80:0xFF]
    assert np.array_equal(neg, -pos)
    # subnormals are integer multiples of 2^-9, normals have 4 significant bits
    assert np.array_equal(v[:8], np.arange(8) / 512.0)
    for x in pos[8:]:
        m, _ = math.frexp(x)
        assert (m * 16).is_integer()


def test_bf16_value_all_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    mine = oracle.bf16_value(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(mine), nan)
    assert np.array_equal(mine[~nan], ref[~nan])
    assert np.array_equal(np.signbit(mine[~nan]), np.signbit(ref[~nan]))


def _exact_bf16_rne(x: float) -> float:
    """Round x to the nearest BF16 value with exact rational arithmetic."""
    if x == 0:
        return x
    fx = Fraction(x)
    sign = -1 if fx < 0 else 1
    a = abs(fx)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    e = max(e, -126)
    q = Fraction(2) ** (e - 7)
    n = a / q
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    r = fl * q
    if r >= Fraction(2) ** 128:
        return sign * math.inf
    return float(sign * r)


def test_bf16_rne_against_exact_rounding():
    rng = np.random.default_rng(7)
    xs = list(rng.standard_normal(3000) * np.exp2(rng.integers(-140, 130, 3000)))
    # exact ties at several binades (even and odd neighbours), subnormal ties, carry into next binade
    for e in (-133, -130, -126, -20, 0, 5, 127):
        for m in (128, 129, 200, 255):
            xs.append(math.ldexp(m + 0.5, e - 7))
    xs += [math.ldexp(255.5, -7), math.ldexp(255.75, 120), 3.3895313892515355e38, 3.4e38, 1e39,
           -1e-45, 5e-324, 1.0 + 2.0 ** -9, 1.0 + 3 * 2.0 ** -9]
    xs = [float(x) for x in xs if math.isfinite(x)]
    got = oracle.bf16_value(oracle.bf16_rne(np.array(xs)))
    for x, g in zip(xs, got):
        want = _exact_bf16_rne(x)
        assert g == want or (g == 0 and want == 0), (x, g, want)
        if want == 0:
            assert math.copysign(1, g) == math.copysign(1, x)


def test_bf16_rne_matches_torch_on_float32_inputs():
    rng = np.random.default_rng(11)
    x = (rng.standard_normal(200000) * np.exp2(rng.integers(-30, 30, 200000))).astype(np.float32)
    mine = oracle.bf16_rne(x.astype(np.float64))
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(mine, ref)


def test_bf16_rne_specials():
    got = oracle.bf16_rne(np.array([0.0, -0.0, np.inf, -np.inf, np.nan, 1.0, -2.0]))
    assert got[0] == 0x0000 and got[1] == 0x8000
    assert got[2] == 0x7F80 and got[3] == 0xFF80
    assert (got[4] & 0x7F80) == 0x7F80 and (got[4] & 0x7F) != 0
    assert got[5] == 0x3F80 and got[6] == 0xC000
