"""Pins of the oracle's whole bank step on tiny banks."""

from fractions import Fraction

import numpy as np

from oracle import BF16, F32, bf16_bits_to_f64, mp_apply_update, muon_bank_step, newton_schulz, recombine, \
    round_fraction, round_to_bf16, step_scalars
from newton_schulz_bank_amd.workloads import WORKLOADS, make_bank, make_random_bank


def _vals(bank, key, dtype):
    a = bank[key]
    return a.astype(np.float64) if dtype == "f32" else bf16_bits_to_f64(a)


def test_dead_slot_stays_exactly_zero():
    bank = make_random_bank(5, 4, 12, 6, dead_slots=(1, 3))
    out = muon_bank_step(_vals(bank, "grad", "bf16"), _vals(bank, "momentum", "bf16"),
                         bank["w_hi"], bank["w_lo"], BF16)
    for s in (1, 3):
        for k in ("momentum", "u", "v64", "v"):
            assert np.all(out[k][s] == 0.0), k
        assert np.all(out["w_hi"][s] == 0) and np.all(out["w_lo"][s] == 0)
    for s in (0, 2):
        assert np.abs(out["v"][s]).max() > 0.05


def test_nesterov_reads_the_stored_buffer():
    """u is formed from the rounded buf' (what g.lerp(buf, mu) reads back), checked
    element by element in exact rationals."""
    bank = make_random_bank(6, 2, 5, 7)
    g = _vals(bank, "grad", "bf16")
    m = _vals(bank, "momentum", "bf16")
    out = muon_bank_step(g, m, bank["w_hi"], bank["w_lo"], BF16)
    sc = out["scalars"]
    for gi, bi, ui in zip(g.ravel(), out["momentum"].ravel(), out["u"].ravel()):
        q = Fraction(sc.nu) * Fraction(float(gi)) + Fraction(sc.mu) * Fraction(float(bi))
        assert round_fraction(q, 8, -126, 127) == ui


def test_step_composes_the_stages():
    bank = make_random_bank(7, 3, 9, 4)
    g = _vals(bank, "grad", "bf16")
    m = _vals(bank, "momentum", "bf16")
    out = muon_bank_step(g, m, bank["w_hi"], bank["w_lo"], BF16, lr=0.05, weight_decay=0.1)
    sc = step_scalars(0.05, 0.1, 0.95, 9, 4)
    assert out["scalars"] == sc
    np.testing.assert_array_equal(out["v64"], newton_schulz(out["u"]))
    np.testing.assert_array_equal(out["v"], round_to_bf16(out["v64"]))
    w_old = recombine(bank["w_hi"], bank["w_lo"]).view(np.float32).astype(np.float64)
    w_new = recombine(out["w_hi"], out["w_lo"]).view(np.float32).astype(np.float64)
    np.testing.assert_allclose(w_new, w_old * sc.decay - sc.eta * out["v"], rtol=1e-6, atol=1e-9)


def test_per_slot_lr_multiplier():
    bank = make_random_bank(8, 3, 6, 6)
    g = _vals(bank, "grad", "bf16")
    m = _vals(bank, "momentum", "bf16")
    per = np.array([1.0, 0.5, 3.0], dtype=np.float32)
    out = muon_bank_step(g, m, bank["w_hi"], bank["w_lo"], BF16, lr_mul_per_slot=per)
    base = muon_bank_step(g, m, bank["w_hi"], bank["w_lo"], BF16)
    np.testing.assert_array_equal(out["w_hi"][0], base["w_hi"][0])
    np.testing.assert_array_equal(out["w_lo"][0], base["w_lo"][0])
    assert out["eta"][1, 0, 0] == base["scalars"].eta * 0.5


def test_per_slot_eta_is_one_fp32_multiply():
    """With a per-slot multiplier m_i the apply uses eta_i = RN32(eta * m_i): one IEEE binary32
    multiply of the two float32 values.  Multipliers whose product with eta is not a float32 (1.1,
    1.7, 0.3) pin the rounding: numpy's own float32 multiply gives the expected value, and the
    weights must be those of the apply with that value, not with the unrounded float64 product."""
    bank = make_random_bank(9, 4, 8, 8)
    g = _vals(bank, "grad", "bf16")
    m = _vals(bank, "momentum", "bf16")
    per = np.array([1.1, 1.7, 0.3, 1.0], dtype=np.float32)
    out = muon_bank_step(g, m, bank["w_hi"], bank["w_lo"], BF16, lr_mul_per_slot=per)
    eta32 = np.float32(out["scalars"].eta)
    want = np.array([np.float32(eta32 * p) for p in per], dtype=np.float64)
    np.testing.assert_array_equal(out["eta"][:, 0, 0], want)
    unrounded = float(eta32) * per.astype(np.float64)
    assert np.count_nonzero(want != unrounded) >= 3, "these multipliers must give inexact products"
    hi, lo = mp_apply_update(bank["w_hi"], bank["w_lo"], out["v"], want[:, None, None], out["scalars"].decay)
    np.testing.assert_array_equal(out["w_hi"], hi)
    np.testing.assert_array_equal(out["w_lo"], lo)
    hi_u, lo_u = mp_apply_update(bank["w_hi"], bank["w_lo"], out["v"], unrounded[:, None, None],
                                 out["scalars"].decay)
    assert not (np.array_equal(hi_u, out["w_hi"]) and np.array_equal(lo_u, out["w_lo"])), \
        "the unrounded product must give other weights on this bank"


def test_fp32_config_zero_momentum_closed_form():
    """The fp32 workload starts from a zero buffer: buf' = RN32(0.05 g) exactly."""
    bank = make_bank(0, 0, slots=[0])
    g = bank["grad"].astype(np.float64)
    out = muon_bank_step(g, np.zeros_like(g), bank["w_hi"], bank["w_lo"], F32)
    sc = out["scalars"]
    np.testing.assert_array_equal(out["momentum"], (sc.nu * g).astype(np.float32).astype(np.float64))
    assert WORKLOADS[0][0].grad_dtype == "f32"


def test_slot_scalar_table_is_applied_per_slot_exactly():
    """With a per-slot table of (mu, nu, decay, eta), slot i's buf', u and weights are the exactly rounded
    values of slot i's own scalars, checked element by element in exact rationals; the scalars are
    arbitrary float32 values (nu need not be 1 - mu)."""
    bank = make_random_bank(10, 3, 4, 5)
    g = _vals(bank, "grad", "bf16")
    m = _vals(bank, "momentum", "bf16")
    tab = np.array([[0.9, 0.1, 0.999, 0.03], [0.95, 0.05, 0.9998, 0.02], [0.8, 0.3, 0.75, 0.011]],
                   dtype=np.float32)
    out = muon_bank_step(g, m, bank["w_hi"], bank["w_lo"], BF16, slot_scalars=tab)
    w_old = recombine(bank["w_hi"], bank["w_lo"]).view(np.float32).astype(np.float64)
    w_new = recombine(out["w_hi"], out["w_lo"]).view(np.float32).astype(np.float64)
    for i in range(3):
        mu, nu, d, eta = (Fraction(float(x)) for x in tab[i])
        for j in np.ndindex(g.shape[1:]):
            b_new = round_fraction(mu * Fraction(float(m[i][j])) + nu * Fraction(float(g[i][j])), 8, -126, 127)
            assert out["momentum"][i][j] == b_new
            u = round_fraction(nu * Fraction(float(g[i][j])) + mu * Fraction(b_new), 8, -126, 127)
            assert out["u"][i][j] == u
            t = round_fraction(Fraction(float(w_old[i][j])) * d, 24, -126, 127)
            r = round_fraction(Fraction(t) - eta * Fraction(float(out["v"][i][j])), 24, -126, 127)
            assert w_new[i][j] == r


def test_slot_scalar_table_with_the_call_scalars_is_the_plain_step():
    """A table that holds the call's own scalars in every slot gives the plain step's bits."""
    bank = make_random_bank(11, 3, 6, 4)
    g = _vals(bank, "grad", "bf16")
    m = _vals(bank, "momentum", "bf16")
    base = muon_bank_step(g, m, bank["w_hi"], bank["w_lo"], BF16)
    sc = base["scalars"]
    tab = np.tile(np.array([[sc.mu, sc.nu, sc.decay, sc.eta]], dtype=np.float32), (3, 1))
    out = muon_bank_step(g, m, bank["w_hi"], bank["w_lo"], BF16, slot_scalars=tab)
    for k in ("momentum", "u", "v", "w_hi", "w_lo"):
        np.testing.assert_array_equal(out[k], base[k])
