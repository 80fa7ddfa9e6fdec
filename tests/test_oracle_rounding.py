"""Pins of the oracle's rounding helpers against brute force and library casts."""

import math
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import bf16_bits_to_f64, f64_to_bf16_bits, round_fraction, round_to_bf16, round_to_f32
from oracle.muon import round_to_format


def _all_finite_bf16_nonneg():
    bits = np.arange(0, 0x7F80, dtype=np.uint16)          # +0 .. largest finite
    return bits, (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _brute_nearest_bf16(x):
    """Nearest non-negative finite bf16 to |x| by search over every bf16 value;
    ties go to the even bit pattern; beyond max+half-ulp gives inf."""
    bits, vals = _all_finite_bf16_nonneg()
    out = np.empty_like(x)
    for i, xi in enumerate(x):
        a = abs(xi)
        j = np.searchsorted(vals, a)
        if j >= len(vals):
            top = vals[-1]
            half_ulp = (vals[-1] - vals[-2]) / 2
            r = math.inf if a >= top + half_ulp else top
        else:
            lo_i, hi_i = max(j - 1, 0), j
            dl, dh = a - vals[lo_i], vals[hi_i] - a
            if dl < dh:
                r = vals[lo_i]
            elif dh < dl:
                r = vals[hi_i]
            else:
                r = vals[lo_i] if bits[lo_i] % 2 == 0 else vals[hi_i]
        out[i] = math.copysign(r, xi)
    return out


def test_bf16_rounding_matches_brute_force_search():
    rng = np.random.default_rng(7)
    x = np.concatenate([
        rng.normal(0, 1, 400),
        rng.normal(0, 1e-3, 400),
        np.ldexp(rng.uniform(0.5, 1, 200), rng.integers(-140, -120, 200)),   # bf16 subnormal range
        np.ldexp(rng.uniform(0.5, 1, 100), rng.integers(120, 128, 100)),     # near the top
    ])
    np.testing.assert_array_equal(round_to_bf16(x), _brute_nearest_bf16(x))


def test_bf16_rounding_ties_go_to_even():
    bits, vals = _all_finite_bf16_nonneg()
    rng = np.random.default_rng(3)
    idx = rng.integers(0, len(vals) - 1, 2000)
    mids = (vals[idx] + vals[idx + 1]) / 2           # exact in float64 (9 significant bits)
    got = round_to_bf16(mids)
    want = np.where(bits[idx] % 2 == 0, vals[idx], vals[idx + 1])
    np.testing.assert_array_equal(got, want)
    np.testing.assert_array_equal(round_to_bf16(-mids), -want)


def test_bf16_rounding_agrees_with_torch_cast_from_fp32():
    """fp32 -> bf16 is a single rounding, so torch's RNE cast is a valid reference."""
    rng = np.random.default_rng(11)
    f = rng.normal(0, 1, 100000).astype(np.float32)
    want = torch.from_numpy(f).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(round_to_bf16(f.astype(np.float64)), want)


def test_f32_rounding_matches_numpy_cast():
    rng = np.random.default_rng(5)
    x = np.concatenate([
        rng.normal(0, 1, 100000),
        np.ldexp(rng.uniform(0.5, 1, 20000), rng.integers(-160, -120, 20000)),   # fp32 subnormals
        np.ldexp(rng.uniform(0.5, 1, 1000), rng.integers(125, 129, 1000)),       # overflow edge
    ])
    with np.errstate(over="ignore"):
        want = x.astype(np.float32).astype(np.float64)
    np.testing.assert_array_equal(round_to_f32(x), want)
    # exact midpoints between neighbouring fp32 values
    f = rng.normal(0, 1, 10000).astype(np.float32)
    nxt = np.nextafter(f, np.float32(np.inf))
    mids = (f.astype(np.float64) + nxt.astype(np.float64)) / 2
    np.testing.assert_array_equal(round_to_f32(mids), mids.astype(np.float32).astype(np.float64))


def test_round_fraction_agrees_with_grid_rounding_and_brute_force():
    rng = np.random.default_rng(9)
    x = np.concatenate([rng.normal(0, 1, 3000), np.ldexp(rng.uniform(-1, 1, 500), rng.integers(-150, -125, 500))])
    for p, emin, emax in ((8, -126, 127), (24, -126, 127)):
        got = np.array([round_fraction(Fraction(float(v)), p, emin, emax) for v in x])
        np.testing.assert_array_equal(got, round_to_format(x, p, emin, emax))
    # a toy format (p=3, emin=-2, emax=2): every rational k/64 in [0, 8) against the enumerated grid
    grid = sorted({m * 2.0 ** (e - 2) for e in range(-2, 3) for m in range(0, 8) if m >= 4 or e == -2})
    grid_bits = {v: i for i, v in enumerate(grid)}   # consecutive values alternate even/odd mantissa
    for k in range(0, 8 * 64):
        q = Fraction(k, 64)
        r = round_fraction(q, 3, -2, 2)
        lo = max(g for g in grid if g <= q)
        his = [g for g in grid if g >= q]
        if not his:
            continue
        hi = min(his)
        if q - Fraction(lo) < Fraction(hi) - q:
            want = lo
        elif q - Fraction(lo) > Fraction(hi) - q:
            want = hi
        else:
            want = lo if grid_bits[lo] % 2 == 0 else hi
        assert r == want, (k, r, want)


def test_bf16_bit_conversions_roundtrip_every_pattern():
    bits = np.arange(0, 65536, dtype=np.uint32).astype(np.uint16)
    vals = bf16_bits_to_f64(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    finite = np.isfinite(ref)
    np.testing.assert_array_equal(vals[finite], ref[finite])
    np.testing.assert_array_equal(np.isnan(vals), np.isnan(ref))
    np.testing.assert_array_equal(f64_to_bf16_bits(vals[finite]), bits[finite])
    with pytest.raises(ValueError):
        f64_to_bf16_bits(np.array([1.0 + 2.0 ** -10]))
