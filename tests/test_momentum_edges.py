"""Momentum + Nesterov on constructed rounding edge cases (tests/momentum_edges.py).

CPU: each case family sits in the regime it is built for, checked in exact rational arithmetic (so the
GPU test below really reaches the tie, sticky-bit and select branches of the correctly rounded sum).
GPU: buf' and u through muon_momentum_update equal the oracle's on every case, bf16 and float32
storage, through the 16-byte vector path (slots of a multiple of 8 elements) and the element-wise one.
"""

import math
from fractions import Fraction

import numpy as np
import pytest

import oracle
from tests import momentum_edges as me


def _is_midpoint(v: Fraction, p: int) -> bool:
    """v is halfway between two neighbouring values of a p-bit binary format (normal range)."""
    if v == 0:
        return False
    a = abs(v)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    q = a / Fraction(2) ** (e - p)          # in [2^p, 2^(p+1)): a midpoint is an odd integer here
    return q.denominator == 1 and q.numerator % 2 == 1


def _regime(x: Fraction, s: float, p: int) -> str:
    """Regime of the exact sum x whose binary64 rounding is s, for a p-bit storage format."""
    if _is_midpoint(x, p):
        return "tie"
    if _is_midpoint(Fraction(s), p):
        return "sticky"
    if p == 8 and _is_midpoint(Fraction(float(np.float32(s))), p):
        return "select"
    return "other"


def _family_regimes(fam, g, b, p, storage):
    want_buf, _ = oracle.momentum_nesterov(g, b, me.MU, me.NU, storage)
    out = {}
    for name, (i0, i1) in fam.items():
        first = second = 0
        for i in range(i0, i1):
            x1 = Fraction(me.MU) * Fraction(b[i]) + Fraction(me.NU) * Fraction(g[i])
            s1 = me.MU * b[i] + me.NU * g[i]
            x2 = Fraction(me.NU) * Fraction(g[i]) + Fraction(me.MU) * Fraction(want_buf[i])
            s2 = me.NU * g[i] + me.MU * want_buf[i]
            kind = name.split()[1] if name.startswith("u ") else name.split()[0]
            if _regime(x1, s1, p) == kind:
                first += 1
            if _regime(x2, s2, 8) == kind:
                second += 1
        out[name] = (first, second, i1 - i0)
    return out


@pytest.mark.parametrize("storage", ["bf16", "f32"])
def test_constructed_cases_reach_their_regimes(storage):
    fam, g, b = me.bf16_cases() if storage == "bf16" else me.f32_cases()
    p = 8 if storage == "bf16" else 24
    reg = _family_regimes(fam, g, b, p, storage)
    for name, (first, second, n) in reg.items():
        kind = name.split()[1] if name.startswith("u ") else name.split()[0]
        if kind not in ("tie", "sticky", "select"):
            continue
        hits = second if name.startswith("u ") else first
        # every direct case, and most of the ones reached through buf' (its first sum must round to the
        # intended buffer value), are in the regime
        need = n if not name.startswith("u ") else n // 2
        assert hits >= need, (name, hits, n)


def test_sticky_cases_differ_from_their_binary64_sum():
    """A sticky case's binary64 sum is the midpoint exactly, while the exact sum is not: rounding the
    binary64 sum alone would take the tie rule and get half of them wrong."""
    fam, g, b = me.bf16_cases()
    wrong = 0
    total = 0
    for name, (i0, i1) in fam.items():
        if not name.startswith("sticky"):
            continue
        for i in range(i0, i1):
            s = me.MU * b[i] + me.NU * g[i]
            x = Fraction(me.MU) * Fraction(b[i]) + Fraction(me.NU) * Fraction(g[i])
            exact = oracle.round_fraction(x, 8, -126, 127)
            naive = oracle.round_fraction(Fraction(s), 8, -126, 127)
            total += 1
            wrong += exact != naive
    assert total > 0 and wrong == total // 2


@pytest.mark.gpu
@pytest.mark.parametrize("storage", ["bf16", "f32"])
@pytest.mark.parametrize("cols", [8, 7])
def test_momentum_edges_bit_exact_on_gpu(storage, cols):
    import torch

    from newton_schulz_bank_amd import api
    from tests.gpu_util import bits, to_dev, vals

    print(f"momentum edges {storage} cols {cols}", flush=True)
    fam, g, b = me.bf16_cases() if storage == "bf16" else me.f32_cases()
    gb = me.as_bank(g, cols, storage)
    bb = me.as_bank(b, cols, storage)
    if cols == 7 and gb.size % 8 == 0:
        raise AssertionError("the element-wise case needs a slot that is not a multiple of 8")
    bf = storage == "bf16"
    dg, db = to_dev(gb, bf), to_dev(bb, bf)
    u = torch.empty(gb.shape, dtype=torch.int16, device="cuda")
    api.muon_momentum_update(dg, db, u, me.MU, me.NU)
    torch.cuda.synchronize()
    want_buf, want_u = oracle.momentum_nesterov(vals(gb), vals(bb), me.MU, me.NU,
                                                oracle.BF16 if bf else oracle.F32)
    got_buf = vals(bits(db)) if bf else db.cpu().numpy().astype(np.float64)
    got_u = vals(bits(u))
    for name, (i0, i1) in fam.items():
        gb_flat, wb_flat = got_buf.ravel()[i0:i1], want_buf.ravel()[i0:i1]
        gu_flat, wu_flat = got_u.ravel()[i0:i1], want_u.ravel()[i0:i1]
        np.testing.assert_array_equal(gb_flat, wb_flat, err_msg=f"buf' {name}")
        np.testing.assert_array_equal(gu_flat, wu_flat, err_msg=f"u {name}")
    assert math.isfinite(float(np.abs(got_u).max()))
