"""Pins of the oracle's mixed-precision apply and the mantissa split/recombine."""

from fractions import Fraction

import numpy as np

from oracle import mp_apply_update, recombine, round_fraction, round_to_bf16, split, step_scalars

F32_FMT = (24, -126, 127)


def test_split_recombine_bijection_exhaustive():
    """recombine(split(x)) == x for all 2**32 patterns (+-0, subnormals, +-inf,
    NaN payloads included).  A map of a finite set onto itself that has a left
    inverse is a bijection, so split(recombine(h, l)) == (h, l) for every pair too."""
    chunk = 1 << 18                      # cache-sized chunks: the sweep takes ~15 s
    base = np.arange(chunk, dtype=np.uint32)
    for start in range(0, 1 << 32, chunk):
        x = base + np.uint32(start)
        hi, lo = split(x)
        assert hi.dtype == np.uint16 and lo.dtype == np.uint16
        if not np.array_equal(recombine(hi, lo), x):
            raise AssertionError(f"round trip fails in chunk starting at {start:#x}")


def test_split_is_a_bit_slice():
    x = np.array([0x3F80FFFF, 0x00000001, 0x80000000, 0x7F800000, 0xFFFFFFFF, 0x12345678], dtype=np.uint32)
    hi, lo = split(x)
    assert list(hi) == [0x3F80, 0x0000, 0x8000, 0x7F80, 0xFFFF, 0x1234]
    assert list(lo) == [0xFFFF, 0x0001, 0x0000, 0x0000, 0xFFFF, 0x5678]
    # the high half is the bf16 truncation of the fp32 master, not its rounding
    f = np.array([1.0 + 2.0 ** -8 + 2.0 ** -20], dtype=np.float32)
    h, _ = split(f.view(np.uint32))
    assert h[0] == 0x3F80


def _exact_apply(hi, lo, v, eta, d):
    w = recombine(hi, lo).view(np.float32).astype(np.float64)
    out_bits = []
    for wi, vi in zip(w, v):
        t = round_fraction(Fraction(float(wi)) * Fraction(d), *F32_FMT)
        r = round_fraction(Fraction(t) - Fraction(eta) * Fraction(float(vi)), *F32_FMT)
        out_bits.append(np.float32(r).view(np.uint32))
    return split(np.array(out_bits, dtype=np.uint32))


def _check_exact(hi, lo, v, eta, d):
    got = mp_apply_update(hi, lo, v, eta, d)
    want = _exact_apply(hi, lo, v, eta, d)
    np.testing.assert_array_equal(got[0], want[0])
    np.testing.assert_array_equal(got[1], want[1])
    return got


def test_apply_is_exactly_rounded_on_random_inputs():
    rng = np.random.default_rng(1)
    sc = step_scalars(0.02, 0.01, 0.95, 768, 768)
    n = 4000
    w = rng.normal(0, 0.02, n).astype(np.float32)
    hi, lo = split(w.view(np.uint32))
    v = round_to_bf16(rng.normal(0, 0.04, n))
    _check_exact(hi, lo, v, sc.eta, sc.decay)


def test_apply_edge_cases():
    sc = step_scalars(0.02, 0.01, 0.95, 3072, 768)
    rng = np.random.default_rng(2)
    # carry across the 16-bit seam: lo = 0xFFFF and the update increases |w|
    hi = np.full(64, 0x3F80, dtype=np.uint16)
    lo = np.full(64, 0xFFFF, dtype=np.uint16)
    v = -round_to_bf16(np.abs(rng.normal(0, 1, 64)))
    h2, l2 = _check_exact(hi, lo, v, sc.eta, 1.0)
    assert np.all(h2 >= 0x3F81)
    # subnormal weights (no flush to zero)
    hi = rng.integers(0, 0x0080, 200).astype(np.uint16)
    lo = rng.integers(0, 65536, 200).astype(np.uint16)
    v = round_to_bf16(rng.normal(0, 1e-40, 200))
    _check_exact(hi, lo, v, sc.eta, sc.decay)
    # cancellation: w close to eta*v so the difference loses most bits
    v = round_to_bf16(rng.normal(0, 0.05, 500))
    w = (np.float64(sc.eta) * v / sc.decay).astype(np.float32)
    hi, lo = split(w.view(np.uint32))
    _check_exact(hi, lo, v, sc.eta, sc.decay)
    # very different magnitudes: exact-rational path of the oracle
    w = rng.normal(0, 1.0, 300).astype(np.float32)
    hi, lo = split(w.view(np.uint32))
    v = round_to_bf16(rng.normal(0, 1e-9, 300))
    _check_exact(hi, lo, v, sc.eta, sc.decay)


def test_apply_identities():
    rng = np.random.default_rng(3)
    w = rng.normal(0, 0.02, 1000).astype(np.float32)
    hi, lo = split(w.view(np.uint32))
    zero = np.zeros(1000)
    h, l = mp_apply_update(hi, lo, zero, 0.02, 1.0)             # v = 0, d = 1: bit-identical
    np.testing.assert_array_equal(h, hi)
    np.testing.assert_array_equal(l, lo)
    sc = step_scalars(0.02, 0.01, 0.95, 768, 768)
    v = round_to_bf16(rng.normal(0, 1, 1000))
    h, l = mp_apply_update(hi, lo, v, 0.0, sc.decay)             # eta = 0: RN32(w*d)
    want = (w.astype(np.float64) * sc.decay).astype(np.float32).view(np.uint32)
    np.testing.assert_array_equal(recombine(h, l), want)
    # all-zero slot stays all-zero
    z16 = np.zeros(100, dtype=np.uint16)
    h, l = mp_apply_update(z16, z16, np.zeros(100), sc.eta, sc.decay)
    assert np.all(h == 0) and np.all(l == 0)


def test_apply_per_slot_eta_broadcast():
    rng = np.random.default_rng(4)
    w = rng.normal(0, 0.02, (3, 4, 5)).astype(np.float32)
    hi, lo = split(w.view(np.uint32))
    v = round_to_bf16(rng.normal(0, 0.04, (3, 4, 5)))
    etas = np.array([0.02, 0.04, 0.03], dtype=np.float32).astype(np.float64)
    d = float(np.float32(0.9998))
    h, l = mp_apply_update(hi, lo, v, etas[:, None, None], d)
    for i in range(3):
        hs, ls = mp_apply_update(hi[i], lo[i], v[i], etas[i], d)
        np.testing.assert_array_equal(h[i], hs)
        np.testing.assert_array_equal(l[i], ls)
