"""GPU (HIP, through the C ABI) against the CPU oracle, stage by stage.

Bars: bit-exact for momentum/u (both sides round the exact value once), for
the mantissa split/recombine and for the apply (both sides compute
RN32(RN32(w*d) - eta*v) exactly); relative Frobenius error <= 3e-2 per slot
for the bf16 Newton-Schulz output against the fp64 oracle on the same bf16
input; dead slots exactly zero.
"""

import sys

import numpy as np
import pytest
import torch

import oracle
from newton_schulz_bank_amd import api
from newton_schulz_bank_amd.workloads import conditioned_bf16_matrices, make_random_bank, random_bf16_matrices
from tests.gpu_util import bits, rel_fro, to_dev, vals

pytestmark = pytest.mark.gpu

NS_TOL = 3e-2


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    api.lib()
    api.mb_device_fault(clear=True)


def assert_no_wait_fault():
    """No dependency wait of a persistent launch gave up at its time cap (which would leave undefined
    values in the affected slots)."""
    torch.cuda.synchronize()
    assert not api.mb_device_fault(), "a persistent Newton-Schulz launch gave up a dependency wait"


# ---------------------------------------------------------------------------
# apply
# ---------------------------------------------------------------------------

APPLY_SHAPES = [(3, 64, 64), (2, 37, 11), (1, 1, 12), (5, 128, 200), (40, 768, 768), (3, 1, 1)]


@pytest.mark.parametrize("shape", APPLY_SHAPES)
@pytest.mark.parametrize("per_slot", [False, True])
def test_apply_bit_exact(shape, per_slot):
    say(f"apply {shape} per_slot={per_slot}")
    rng = np.random.default_rng(sum(shape) + per_slot)
    w = rng.normal(0, 0.02, shape).astype(np.float32)
    hi, lo = oracle.split(w.view(np.uint32))
    v64 = oracle.round_to_bf16(rng.normal(0, 0.04, shape))
    v = oracle.f64_to_bf16_bits(v64)
    sc = oracle.step_scalars(0.02, 0.01, 0.95, shape[1], shape[2])
    per = rng.uniform(0.5, 2.0, shape[0]).astype(np.float32) if per_slot else None
    eta = oracle.round_to_f32(sc.eta * per.astype(np.float64))[:, None, None] if per_slot else sc.eta
    want_hi, want_lo = oracle.mp_apply_update(hi, lo, v64, eta, sc.decay)
    d_hi, d_lo, d_v = to_dev(hi), to_dev(lo), to_dev(v)
    api.mp_apply_update(d_hi, d_lo, d_v, sc.eta, sc.decay, to_dev(per) if per_slot else None)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(d_hi), want_hi)
    np.testing.assert_array_equal(bits(d_lo), want_lo)


def test_apply_edge_patterns():
    """Carry across the 16-bit seam, subnormal weights, cancellation, zeros."""
    say("apply edge patterns")
    rng = np.random.default_rng(5)
    n = 4096
    hi = np.concatenate([np.full(1024, 0x3F80), rng.integers(0, 0x80, 1024), rng.integers(0, 0x8000, 1024),
                         np.zeros(1024)]).astype(np.uint16)
    lo = np.concatenate([np.full(1024, 0xFFFF), rng.integers(0, 65536, 2048), np.zeros(1024)]).astype(np.uint16)
    v64 = np.concatenate([-oracle.round_to_bf16(np.abs(rng.normal(0, 1, 1024))),
                          oracle.round_to_bf16(rng.normal(0, 1e-39, 1024)),
                          oracle.round_to_bf16(rng.normal(0, 0.05, 1024)), np.zeros(1024)])
    # cancellation block: w = eta*v/decay rounded, in the third quarter
    sc = oracle.step_scalars(0.02, 0.01, 0.95, 3072, 768)
    wc = (np.float64(sc.eta) * v64[2048:3072] / sc.decay).astype(np.float32)
    hi[2048:3072], lo[2048:3072] = oracle.split(wc.view(np.uint32))
    v = oracle.f64_to_bf16_bits(v64)
    want = oracle.mp_apply_update(hi, lo, v64, sc.eta, sc.decay)
    d_hi, d_lo = to_dev(hi.reshape(1, 1, n)), to_dev(lo.reshape(1, 1, n))
    api.mp_apply_update(d_hi, d_lo, to_dev(v.reshape(1, 1, n)), sc.eta, sc.decay)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits(d_hi).ravel(), want[0])
    np.testing.assert_array_equal(bits(d_lo).ravel(), want[1])
    assert np.all(bits(d_hi).ravel()[3072:] == 0) and np.all(bits(d_lo).ravel()[3072:] == 0)


# ---------------------------------------------------------------------------
# momentum + Nesterov
# ---------------------------------------------------------------------------

MOM_CASES = [((4, 256, 256), "f32"), ((3, 64, 64), "f32"), ((5, 33, 17), "bf16"), ((2, 128, 96), "bf16"),
             ((3, 7, 5), "f32"), ((40, 768, 768), "bf16")]


@pytest.mark.parametrize("shape,dtype", MOM_CASES)
def test_momentum_bit_exact(shape, dtype):
    say(f"momentum {shape} {dtype}")
    scale = 1.0 if dtype == "f32" else 1e-3
    bank = make_random_bank(sum(shape), *shape, grad_dtype=dtype, grad_scale=scale, mom_scale=scale)
    sc = oracle.step_scalars(0.02, 0.01, 0.95, shape[1], shape[2])
    want_buf, want_u = oracle.momentum_nesterov(vals(bank["grad"]), vals(bank["momentum"]), sc.mu, sc.nu,
                                                oracle.F32 if dtype == "f32" else oracle.BF16)
    bf = dtype == "bf16"
    g, m = to_dev(bank["grad"], bf), to_dev(bank["momentum"], bf)
    u = torch.empty(shape, dtype=torch.int16, device="cuda")
    api.muon_momentum_update(g, m, u, sc.mu, sc.nu)
    torch.cuda.synchronize()
    got_buf = m.cpu().numpy().astype(np.float64) if dtype == "f32" else vals(bits(m))
    np.testing.assert_array_equal(got_buf, want_buf)
    np.testing.assert_array_equal(vals(bits(u)), want_u)


# ---------------------------------------------------------------------------
# Newton-Schulz
# ---------------------------------------------------------------------------

NS_SHAPES = [(4, 256, 256), (3, 100, 260), (3, 260, 100), (2, 130, 130), (2, 64, 512), (2, 512, 64),
             (2, 1, 12), (3, 6, 12), (2, 12, 6), (2, 768, 768), (1, 3072, 768), (1, 768, 3072), (1, 1024, 1024),
             (1, 200, 8), (2, 257, 129),
             # one workgroup per slot for every round (Gram side <= 64, <= 4096 elements)
             (16, 1, 12), (16, 6, 12), (2, 64, 64), (3, 40, 3), (2, 16, 256), (2, 256, 16),
             # degenerate slots: a scalar, a row and a column of two
             (3, 1, 1), (2, 1, 2), (2, 2, 1)]


@pytest.mark.parametrize("shape", NS_SHAPES)
def test_ns_parity(shape):
    say(f"ns {shape}")
    x = random_bf16_matrices(1 + sum(shape), *shape, scale=1e-3)
    want = oracle.newton_schulz(vals(x))
    y = api.ns_orthogonalize_batched(to_dev(x))
    torch.cuda.synchronize()
    got = vals(bits(y))
    err = rel_fro(got, want)
    say(f"  rel err per slot: {np.array2string(err, precision=4)}")
    assert np.all(err <= NS_TOL), err


def test_ns_zero_slot_and_determinism():
    say("ns zero slot / determinism")
    x = random_bf16_matrices(3, 4, 256, 384, scale=1.0)
    x[2] = 0
    dx = to_dev(x)
    y1 = bits(api.ns_orthogonalize_batched(dx))
    y2 = bits(api.ns_orthogonalize_batched(dx))
    torch.cuda.synchronize()
    assert np.all(y1[2] == 0)
    np.testing.assert_array_equal(y1, y2)


@pytest.mark.parametrize("shape", [(2, 128, 192), (3, 6, 12)])
def test_ns_in_place(shape):
    say(f"ns in place {shape}")
    x = random_bf16_matrices(4, *shape)
    for steps in (5, 1):
        dx = to_dev(x)
        ref = bits(api.ns_orthogonalize_batched(dx, steps=steps))
        api.ns_orthogonalize_batched(dx, dx, steps=steps)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(bits(dx), ref)


def test_ns_band_on_well_conditioned_inputs():
    """Singular values of the output lie in the iteration's fixed band [0.6818, 1.1344], widened by 0.03."""
    say("ns band")
    for shape in [(4, 256, 256), (2, 128, 384), (2, 384, 128)]:
        x = conditioned_bf16_matrices(sum(shape), *shape)
        got = vals(bits(api.ns_orthogonalize_batched(to_dev(x))))
        for i in range(shape[0]):
            sv = np.linalg.svd(got[i], compute_uv=False)
            assert sv.min() >= 0.6818 - 0.03 and sv.max() <= 1.1344 + 0.03, (shape, sv.min(), sv.max())


def test_ns_transpose_equivariance():
    say("ns transpose equivariance")
    x = random_bf16_matrices(8, 3, 192, 320)
    y = vals(bits(api.ns_orthogonalize_batched(to_dev(x))))
    xt = np.ascontiguousarray(x.transpose(0, 2, 1))
    yt = vals(bits(api.ns_orthogonalize_batched(to_dev(xt))))
    assert np.all(rel_fro(yt.transpose(0, 2, 1), y) <= NS_TOL)


# ---------------------------------------------------------------------------
# Newton-Schulz: persistent (one launch per bank) vs one launch per contraction
# ---------------------------------------------------------------------------
# Both schedules run the same tile arithmetic with the same per-element k order
# (MFMA blocks of 16 in increasing k) and the same epilogue, so their outputs
# must agree bit for bit; the oracle bound is checked as well.

PERSIST_SHAPES = [(8, 256, 256), (3, 256, 256), (17, 256, 256), (9, 256, 512), (5, 512, 256), (2, 768, 768),
                  (1, 256, 1024), (2, 1024, 256), (3, 768, 1280),
                  # sides multiples of 256, short side >= 512 and more than 8 slots: 256x256 tiles (8 or
                  # fewer slots take 128x128 tiles, as the shapes above and (8, 512, 512) do)
                  (9, 512, 512), (8, 512, 512), (16, 512, 512), (17, 512, 768), (16, 1024, 512),
                  # sides multiples of 128 but not of 256: 128x128 tiles, two workgroups per CU
                  (6, 384, 384), (9, 128, 128), (3, 128, 640), (2, 640, 384)]


def _ns_per_round(dx, **kw):
    prev = api.mb_ns_set_path(1)
    try:
        return bits(api.ns_orthogonalize_batched(dx, **kw))
    finally:
        api.mb_ns_set_path(prev)


@pytest.mark.parametrize("shape", PERSIST_SHAPES)
def test_ns_persistent_bitwise_and_oracle(shape):
    say(f"ns persistent {shape}")
    x = random_bf16_matrices(7 + sum(shape), *shape, scale=1e-3)
    if shape[0] >= 3:
        x[1] = 0      # a dead slot inside the batch
    dx = to_dev(x)
    ref = _ns_per_round(dx)
    got = bits(api.ns_orthogonalize_batched(dx))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(got, ref)
    if shape[0] >= 3:
        assert np.all(got[1] == 0)
    assert_no_wait_fault()
    if shape[1] * shape[2] <= 768 * 768:
        err = rel_fro(vals(got), oracle.newton_schulz(vals(x)))
        say(f"  rel err per slot: {np.array2string(err, precision=4)}")
        assert np.all(err <= NS_TOL), err


@pytest.mark.parametrize("steps", [1, 2, 3])
def test_ns_persistent_steps(steps):
    say(f"ns persistent steps={steps}")
    x = random_bf16_matrices(40 + steps, 6, 256, 512)
    dx = to_dev(x)
    ref = _ns_per_round(dx, steps=steps)
    got = bits(api.ns_orthogonalize_batched(dx, steps=steps))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(got, ref)
    assert_no_wait_fault()


def test_ns_persistent_in_place_and_repeat():
    say("ns persistent in place / repeat")
    x = random_bf16_matrices(50, 10, 512, 256)
    ref = _ns_per_round(to_dev(x))
    for steps in (5, 1):
        want = _ns_per_round(to_dev(x), steps=steps)
        dx = to_dev(x)
        api.ns_orthogonalize_batched(dx, dx, steps=steps)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(bits(dx), want)
    # the same workspace reused by back-to-back calls on one stream
    dx = to_dev(x)
    ws = torch.empty(api.lib().mb_ns_workspace_bytes(*x.shape), dtype=torch.uint8, device="cuda")
    outs = [api.ns_orthogonalize_batched(dx, workspace=ws) for _ in range(3)]
    torch.cuda.synchronize()
    for o in outs:
        np.testing.assert_array_equal(bits(o), ref)
    assert_no_wait_fault()


# ---------------------------------------------------------------------------
# Newton-Schulz with per-round coefficients
# ---------------------------------------------------------------------------

SCHEDULE = [(3.4445, -4.7750, 2.0315), (3.0, -3.2, 1.2), (2.0, -1.5, 0.5), (1.875, -1.25, 0.375), (1.5, -0.5, 0.0)]


@pytest.mark.parametrize("shape", [(4, 256, 256), (3, 768, 256), (5, 384, 384), (2, 100, 260), (3, 6, 12)])
def test_ns_schedule_parity(shape):
    say(f"ns schedule {shape}")
    x = random_bf16_matrices(60 + sum(shape), *shape, scale=1e-3)
    want = oracle.newton_schulz(vals(x), schedule=SCHEDULE)
    dx = to_dev(x)
    got = bits(api.ns_orthogonalize_batched(dx, schedule=SCHEDULE))
    torch.cuda.synchronize()
    err = rel_fro(vals(got), want)
    say(f"  rel err per slot: {np.array2string(err, precision=4)}")
    assert np.all(err <= NS_TOL), err
    b, r, c = shape
    if min(r, c) > 64 or r * c > 4096:
        # the tile kernels of both schedules give the same bits; small slots (Gram side <= 64, <= 4096
        # elements) take the small-slot kernel on one and the generic tiles on the other
        np.testing.assert_array_equal(got, _ns_per_round(dx, schedule=SCHEDULE))
    else:
        err1 = rel_fro(vals(_ns_per_round(dx, schedule=SCHEDULE)), want)
        assert np.all(err1 <= NS_TOL), err1


def test_ns_constant_schedule_equals_plain_call():
    say("ns constant schedule")
    x = random_bf16_matrices(70, 4, 256, 512)
    dx = to_dev(x)
    plain = bits(api.ns_orthogonalize_batched(dx))
    sched = bits(api.ns_orthogonalize_batched(dx, schedule=[(3.4445, -4.7750, 2.0315)] * 5))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(plain, sched)


def test_bank_step_with_schedule():
    say("bank step with schedule")
    bank = make_random_bank(71, 3, 256, 384)
    dev = api.Bank(grad=to_dev(bank["grad"], True), momentum=to_dev(bank["momentum"], True), w_hi=to_dev(bank["w_hi"]),
                   w_lo=to_dev(bank["w_lo"]))
    dev.v_out = torch.empty(bank["w_hi"].shape, dtype=torch.int16, device="cuda")
    dev.u_out = torch.empty(bank["w_hi"].shape, dtype=torch.int16, device="cuda")
    api.muon_bank_step([dev], hp=api.make_hparams(schedule=SCHEDULE))
    torch.cuda.synchronize()
    u = vals(bits(dev.u_out))
    want_v = oracle.newton_schulz(u, schedule=SCHEDULE)
    err = rel_fro(vals(bits(dev.v_out)), want_v)
    assert np.all(err <= NS_TOL), err
    sc = oracle.step_scalars(0.02, 0.01, 0.95, 256, 384)
    want_hi, want_lo = oracle.mp_apply_update(bank["w_hi"], bank["w_lo"], vals(bits(dev.v_out)), sc.eta, sc.decay)
    np.testing.assert_array_equal(bits(dev.w_hi), want_hi)
    np.testing.assert_array_equal(bits(dev.w_lo), want_lo)
