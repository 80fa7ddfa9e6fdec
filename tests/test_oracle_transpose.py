"""Pins of the transpose oracle: brute force, library routines and exact rationals."""

from fractions import Fraction

import numpy as np
import torch

import oracle
from oracle import transpose_add, transpose_copy


def test_copy_is_the_transpose_by_brute_force_and_numpy():
    rng = np.random.default_rng(1)
    for shape in [(1, 1), (1, 12), (7, 3), (37, 64), (64, 129)]:
        x = rng.integers(0, 65536, shape).astype(np.uint16)
        y = transpose_copy(x)
        assert y.shape == shape[::-1] and y.dtype == x.dtype
        for i in range(shape[0]):
            for j in range(shape[1]):
                assert y[j, i] == x[i, j]
        np.testing.assert_array_equal(y, np.transpose(x))
        np.testing.assert_array_equal(transpose_copy(y), x)


def _exact_rn(a, b, p):
    """Correctly rounded a + b (normal range) to p significand bits, round half to even."""
    return oracle.round_fraction(Fraction(float(a)) + Fraction(float(b)), p, -1000, 1000)


def _edge_f32(rng, n):
    a = rng.normal(0, 1, n).astype(np.float32)
    b = rng.normal(0, 1, n).astype(np.float32)
    b[: n // 4] = (a[: n // 4] * np.float32(2.0 ** -30)).astype(np.float32)   # far apart exponents
    b[n // 4: n // 2] = -a[n // 4: n // 2]                                      # exact cancellation
    b[n // 2: n // 2 + 8] = np.float32(0)
    return a, b


def test_add_f32_is_the_correctly_rounded_sum():
    rng = np.random.default_rng(2)
    a, b = _edge_f32(rng, 4000)
    dst, src = a.reshape(40, 100), b.reshape(100, 40).copy()
    src[:] = b.reshape(40, 100).T        # src^T lines up with dst
    got = transpose_add(dst, src, oracle.F32)
    flat_got = got.ravel()
    for k in range(0, 4000, 7):
        want = _exact_rn(a[k], b[k], 24)
        assert float(flat_got[k]) == want, (k, a[k], b[k])
    # the library's own float32 addition rounds once too
    lib = (torch.from_numpy(dst) + torch.from_numpy(src).T).numpy()
    np.testing.assert_array_equal(got, lib)
    # adding zeros changes nothing (bits), including signed zeros of dst
    np.testing.assert_array_equal(transpose_add(dst, np.zeros_like(src), oracle.F32).view(np.uint32),
                                  (dst + np.float32(0)).view(np.uint32))


def test_add_bf16_is_the_correctly_rounded_sum():
    rng = np.random.default_rng(3)
    n = 3000
    a = oracle.round_to_bf16(rng.normal(0, 1, n))
    b = oracle.round_to_bf16(rng.normal(0, 1, n))
    b[:300] = oracle.round_to_bf16(a[:300] * 2.0 ** -20)   # far apart exponents
    b[300:600] = -a[300:600]
    ab, bb = oracle.f64_to_bf16_bits(a), oracle.f64_to_bf16_bits(b)
    dst, src = ab.reshape(30, 100), bb.reshape(30, 100).T.copy()
    got = oracle.bf16_bits_to_f64(transpose_add(dst, src, oracle.BF16)).ravel()
    for k in range(0, n, 5):
        assert got[k] == _exact_rn(a[k], b[k], 8), (k, a[k], b[k])
    lib = (torch.from_numpy(dst.view(np.int16)).view(torch.bfloat16).float() +
           torch.from_numpy(src.view(np.int16)).view(torch.bfloat16).float().T).to(torch.bfloat16)
    np.testing.assert_array_equal(transpose_add(dst, src, oracle.BF16), lib.view(torch.int16).numpy().view(np.uint16))
