"""Newton-Schulz far from the gradients' scale, through the C ABI.

The Frobenius scale 1 / (||X||_F + eps) is taken once per slot before the
first round ("Muon Custom Sizing", section 2.3 asks for the norm scaling
first), so the result depends on the input's scale only through eps.  The GPU
folds the scale into the first round's epilogues while the slot's norm is in
a safe range and reads an exact power-of-two copy of the slot outside it.
These tests hold it to the oracle at input scales from 1e-30 to 1e30, and to
exact scale invariance (bit for bit) with eps = 0 and power-of-two scales,
where every rounding of both routes scales exactly.
"""

import numpy as np
import pytest
import torch

import oracle
from newton_schulz_bank_amd import api
from newton_schulz_bank_amd.workloads import make_random_bank, random_bf16_matrices
from tests.gpu_util import bits, rel_fro, to_dev, vals

pytestmark = pytest.mark.gpu

NS_TOL = 3e-2
# persistent launch (128-tiles), tall persistent slots, ragged (per-contraction kernels), small slots
SHAPES = [(8, 768, 768), (3, 3072, 768), (2, 100, 260), (4, 6, 12)]


def _ns(x_bits, eps=1e-7):
    y = api.ns_orthogonalize_batched(to_dev(x_bits), eps=eps)
    torch.cuda.synchronize()
    return bits(y)


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_ns_matches_oracle_at_every_scale(shape):
    b, r, c = shape
    print(f"scales {shape}", flush=True)
    for i, sigma in enumerate((1e-33, 1e-15, 1e-9, 1e-1, 1e9, 1e27)):
        x = random_bf16_matrices(5200 + i, b, r, c, sigma)
        got = vals(_ns(x))
        want = oracle.newton_schulz(vals(x))
        err = rel_fro(got, want)
        print(f"  sigma {sigma:g}: max rel err {err.max():.5f}", flush=True)
        assert np.all(np.isfinite(got))
        assert np.all(err <= NS_TOL), (sigma, err)


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_ns_bits_are_scale_invariant_without_eps(shape):
    """With eps = 0, NS(2^j X) has the bits of NS(X): inside the folded range every product, sum and
    scale is multiplied by an exact power of two, and outside it the pre-scaled copy of 2^j X is the
    same bf16 matrix as that of X.  Scales 2^-90 and 2^90 take the pre-scaled route, 2^-50 too; 2^0
    and 2^50 the folded one.  The oracle agrees within the tolerance with eps = 0 as well."""
    b, r, c = shape
    x = random_bf16_matrices(5300, b, r, c, 1e-3)
    x64 = vals(x)
    nz = np.abs(x64[x64 != 0])
    ref = _ns(x, eps=0.0)
    err = rel_fro(vals(ref), oracle.newton_schulz(x64, eps=0.0))
    assert np.all(err <= NS_TOL), err
    for j in (-90, -50, 50, 90):
        # the scaled matrix must be exact: every element stays a normal bf16 value
        assert nz.min() * 2.0 ** j >= 2.0 ** -126 and nz.max() * 2.0 ** j < 2.0 ** 127
        xs = oracle.f64_to_bf16_bits(x64 * 2.0 ** j)
        got = _ns(xs, eps=0.0)
        diff = np.nonzero(np.any(got != ref, axis=(1, 2)))[0]
        assert diff.size == 0, f"2^{j}: slots {diff.tolist()} differ from the unscaled input's bits"


def test_single_subnormal_element_is_live():
    """A slot whose one nonzero element is a bf16 subnormal (2^-130) is live: its sum of squares is
    nonzero, and the result is the oracle's (eps = 1e-7 dominates, so the map is nearly linear), not
    zero.  With eps = 0 it is a unit-norm input: the one singular value 1 goes to p^5(1)."""
    for eps in (1e-7, 0.0):
        for shape in ((2, 768, 768), (2, 6, 12), (2, 100, 260)):
            x = np.zeros(shape, dtype=np.uint16)
            x[0, 3, 5] = oracle.f64_to_bf16_bits(np.array([2.0 ** -130]))[0]
            got = vals(_ns(x, eps=eps))
            want = oracle.newton_schulz(vals(x[:1]), eps=eps)
            assert np.count_nonzero(got[0]) == 1 and got[0, 3, 5] > 0, (eps, shape)
            assert np.all(got[1] == 0)
            assert rel_fro(got[:1], want[:1])[0] <= NS_TOL, (eps, shape)


def test_bank_step_with_slots_of_very_different_scales():
    """One bank whose slots hold gradients and momenta at 1e-3, 1e-36, 1e25 and zero: momentum, u and the
    apply bit-exact, Newton-Schulz within the tolerance on every live slot, the zero slot exactly zero."""
    scales = (1e-3, 1e-36, 1e25, None)
    parts = []
    for i, sc in enumerate(scales):
        if sc is None:
            parts.append(make_random_bank(5400 + i, 1, 768, 768, dead_slots=(0,)))
        else:
            parts.append(make_random_bank(5400 + i, 1, 768, 768, grad_scale=sc, mom_scale=sc))
    h = {k: np.concatenate([p[k] for p in parts]) for k in parts[0]}
    b = api.Bank(grad=to_dev(h["grad"], True), momentum=to_dev(h["momentum"], True), w_hi=to_dev(h["w_hi"]),
                 w_lo=to_dev(h["w_lo"]))
    b.v_out = torch.empty(h["w_hi"].shape, dtype=torch.int16, device="cuda")
    b.u_out = torch.empty(h["w_hi"].shape, dtype=torch.int16, device="cuda")
    api.mb_device_fault(clear=True)
    api.muon_bank_step([b])
    torch.cuda.synchronize()
    assert not api.mb_device_fault()
    sc = oracle.step_scalars(0.02, 0.01, 0.95, 768, 768)
    want_buf, want_u = oracle.momentum_nesterov(vals(h["grad"]), vals(h["momentum"]), sc.mu, sc.nu, oracle.BF16)
    np.testing.assert_array_equal(vals(bits(b.momentum)), want_buf)
    u = bits(b.u_out)
    np.testing.assert_array_equal(vals(u), want_u)
    v = bits(b.v_out)
    err = rel_fro(vals(v[:3]), oracle.newton_schulz(vals(u[:3])))
    print(f"  per-slot NS rel err {err}", flush=True)
    assert np.all(err <= NS_TOL), err
    assert np.all(v[3] == 0)
    hi, lo = oracle.mp_apply_update(h["w_hi"], h["w_lo"], vals(v), sc.eta, sc.decay)
    np.testing.assert_array_equal(bits(b.w_hi), hi)
    np.testing.assert_array_equal(bits(b.w_lo), lo)
