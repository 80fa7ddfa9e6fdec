"""Pins of the oracle's momentum / Nesterov stage and host scalars."""

import json
import math
import os
from fractions import Fraction

import numpy as np
import torch

from oracle import BF16, F32, momentum_nesterov, round_fraction, round_to_bf16, round_to_f32, step_scalars
from tests.conftest import GOLDEN

F32_FMT = (24, -126, 127)
BF16_FMT = (8, -126, 127)


def _bf16_values(rng, n, scale):
    return round_to_bf16(rng.normal(0, scale, n))


def _exact(c1, x1, c2, x2, fmt):
    return np.array([round_fraction(Fraction(c1) * Fraction(float(a)) + Fraction(c2) * Fraction(float(b)), *fmt)
                     for a, b in zip(x1, x2)])


def test_momentum_is_exactly_rounded_bf16():
    rng = np.random.default_rng(1)
    sc = step_scalars(0.02, 0.01, 0.95, 768, 768)
    g = _bf16_values(rng, 3000, 1e-3)
    buf = _bf16_values(rng, 3000, 1e-3)
    # force some huge exponent gaps so the exact-rational path is taken
    g[:50] = round_to_bf16(rng.normal(0, 1e-12, 50))
    buf[50:100] = round_to_bf16(rng.normal(0, 1e-14, 50))
    buf_new, u = momentum_nesterov(g, buf, sc.mu, sc.nu, BF16)
    np.testing.assert_array_equal(buf_new, _exact(sc.mu, buf, sc.nu, g, BF16_FMT))
    np.testing.assert_array_equal(u, _exact(sc.nu, g, sc.mu, buf_new, BF16_FMT))


def test_momentum_is_exactly_rounded_fp32():
    rng = np.random.default_rng(2)
    sc = step_scalars(0.02, 0.01, 0.95, 256, 256)
    g = round_to_f32(rng.normal(0, 1, 2000))
    buf = round_to_f32(rng.normal(0, 1, 2000))
    buf_new, u = momentum_nesterov(g, buf, sc.mu, sc.nu, F32)
    np.testing.assert_array_equal(buf_new, _exact(sc.mu, buf, sc.nu, g, F32_FMT))
    np.testing.assert_array_equal(u, _exact(sc.nu, g, sc.mu, buf_new, BF16_FMT))


def test_momentum_closed_forms():
    rng = np.random.default_rng(3)
    g = round_to_f32(rng.normal(0, 1, 1000))
    sc = step_scalars(0.02, 0.01, 0.95, 256, 256)
    # zero buffer: buf' = RN(nu*g)
    buf_new, u = momentum_nesterov(g, np.zeros_like(g), sc.mu, sc.nu, F32)
    np.testing.assert_array_equal(buf_new, round_to_f32(sc.nu * g))
    # u = RN_bf16((1-mu)(1+mu) g) up to the rounding of buf'; 0.0975*g within 2 bf16 ulps
    np.testing.assert_allclose(u, 0.0975 * g, rtol=2 ** -7, atol=0)
    # mu = 0: plain copy of the gradient; mu = 1: the old buffer
    buf = round_to_f32(rng.normal(0, 1, 1000))
    b0, u0 = momentum_nesterov(g, buf, 0.0, 1.0, F32)
    np.testing.assert_array_equal(b0, g)
    np.testing.assert_array_equal(u0, round_to_bf16(g))
    b1, u1 = momentum_nesterov(g, buf, 1.0, 0.0, F32)
    np.testing.assert_array_equal(b1, buf)
    np.testing.assert_array_equal(u1, round_to_bf16(buf))


def test_momentum_follows_torch_lerp_semantics():
    """The pages state the step as buf.lerp_(g, 1-mu) and g.lerp(buf, mu); torch's
    lerp in float64 is the library routine that defines them.  Agreement to fp32
    rounding pins the operand order and which weight goes where."""
    rng = np.random.default_rng(4)
    mu = 0.95
    sc = step_scalars(0.02, 0.01, mu, 64, 64)
    g = round_to_f32(rng.normal(0, 1, 5000))
    buf = round_to_f32(rng.normal(0, 1, 5000))
    tb = torch.from_numpy(buf.copy())
    tg = torch.from_numpy(g.copy())
    tb.lerp_(tg, 1 - mu)
    tu = tg.lerp(tb, mu)
    buf_new, u = momentum_nesterov(g, buf, sc.mu, sc.nu, F32)
    np.testing.assert_allclose(buf_new, tb.numpy(), rtol=1e-6, atol=1e-7)
    np.testing.assert_allclose(u, tu.numpy(), rtol=2 ** -7, atol=1e-7)


def test_momentum_many_steps_is_an_ema():
    """k steps from a zero buffer: buf_k = (1-mu) * sum_j mu^(k-j) g_j."""
    rng = np.random.default_rng(5)
    sc = step_scalars(0.02, 0.01, 0.9, 8, 8)
    gs = [round_to_f32(rng.normal(0, 1, 500)) for _ in range(12)]
    buf = np.zeros(500)
    for gk in gs:
        buf, _ = momentum_nesterov(gk, buf, sc.mu, sc.nu, F32)
    k = len(gs)
    ema = sum((1 - 0.9) * 0.9 ** (k - 1 - j) * gs[j] for j in range(k))
    np.testing.assert_allclose(buf, ema, rtol=1e-5, atol=1e-6)


def test_step_scalars_closed_forms():
    d = json.load(open(os.path.join(GOLDEN, "muon_defaults.json")))
    lr, wd, mu = d["lr"], d["weight_decay"], d["momentum"]
    f32 = lambda v: float(np.float32(v))
    sq = step_scalars(lr, wd, mu, 768, 768)
    assert sq.mu == f32(0.95) and sq.nu == f32(0.05000000000000004)
    assert sq.decay == f32(1 - 0.0002) and sq.eta == f32(0.02)
    assert step_scalars(lr, wd, mu, 3072, 768).eta == f32(0.04)            # sqrt(4) = 2
    assert step_scalars(lr, wd, mu, 4096, 1024).eta == f32(0.04)
    assert step_scalars(lr, wd, mu, 768, 3072).eta == f32(0.02)            # wide: max(1, .) = 1
    assert step_scalars(lr, wd, mu, 1, 12).eta == f32(0.02)
    assert step_scalars(lr, wd, mu, 6, 12).eta == f32(0.02)
    e2816 = step_scalars(lr, wd, mu, 2816, 768).eta
    assert abs(e2816 / 0.02 - 1.914854) < 1e-6                              # sqrt(2816/768)
    assert step_scalars(lr, wd, mu, 768, 768, lr_mul=2.0, wd_mul=3.0).decay == f32(1 - 0.02 * 0.01 * 3.0)
    assert step_scalars(lr, wd, mu, 768, 768, lr_mul=2.0).eta == f32(0.04)
    assert math.isclose(sq.mu + sq.nu, 1.0, abs_tol=1e-7)
