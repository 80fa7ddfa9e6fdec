"""The whole Muon bank step on the five workloads, through muon_bank_step.

Stage isolation: the oracle's momentum runs on the same inputs (bit-exact
buf' and u), the oracle's Newton-Schulz on the GPU's u (tolerance), and the
oracle's apply on the GPU's v (bit-exact weights), so no stage's tolerance
leaks into the next.  End to end, the weights agree within one fp32 ulp plus
eta times the difference of the two v.  The big workloads are checked on
sampled slots (plus every dead slot); Newton-Schulz is compared with the
oracle on every live slot, except on the 350M banks' two large banks (both
readings of the dead 2816 slot), where eight slots cover the eight XCD queues.  The launch configuration is the one
the benchmark times.
"""

import functools
import sys

import numpy as np
import pytest
import torch

import oracle
from newton_schulz_bank_amd import api
from newton_schulz_bank_amd.workloads import WORKLOADS, make_bank
from tests.gpu_util import bits, rel_fro, to_dev, vals

pytestmark = pytest.mark.gpu

NS_TOL = 3e-2


def queue_cover(spec):
    """Eight live slots of a bank, one for each residue s mod 8, spread over the bank.  A persistent launch
    numbers the slots of its banks in one sequence and runs slot g on XCD queue g mod 8; every bank of the
    350M workloads starts at a multiple of 8 in that sequence, so these slots meet all eight queues."""
    live = spec.live_slots
    picks = []
    for r in range(8):
        cands = [s for s in live if s % 8 == r]
        if cands:
            picks.append(cands[(r * len(cands)) // 8])
    return picks


# slots checked element by element (None = every slot) and slots whose Newton-Schulz output is compared
# with the oracle's (None = every live slot; "cover" = queue_cover)
SAMPLES = {
    0: {"elem": None, "ns": None},
    1: {"elem": None, "ns": None},
    2: {"elem": None, "ns": None},
    3: {"elem": None, "ns": None},
    4: {"elem": {0: [0, 95], 1: [0, 47], 2: [0, 7, 13, 14, 15, 23]}, "ns": {0: "cover", 1: "cover", 2: None}},
    5: {"elem": None, "ns": None},
    6: {"elem": None, "ns": None},
    7: {"elem": {0: [0], 1: [0], 2: [0, 6, 7, 8, 14, 15, 23]}, "ns": {0: "cover", 1: "cover", 2: None}},
}


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@functools.lru_cache(maxsize=2)
def host_inputs(config):
    return tuple(make_bank(config, i) for i in range(len(WORKLOADS[config])))


def _upload(config):
    specs = WORKLOADS[config]
    banks = []
    for spec, h in zip(specs, host_inputs(config)):
        bf = spec.grad_dtype == "bf16"
        b = api.Bank(grad=to_dev(h["grad"], bf), momentum=to_dev(h["momentum"], bf), w_hi=to_dev(h["w_hi"]),
                     w_lo=to_dev(h["w_lo"]))
        b.v_out = torch.empty(h["w_hi"].shape, dtype=torch.int16, device="cuda")
        b.u_out = torch.empty(h["w_hi"].shape, dtype=torch.int16, device="cuda")
        banks.append(b)
    return banks


def _run(config):
    specs = WORKLOADS[config]
    banks = _upload(config)
    api.muon_bank_step(banks)
    torch.cuda.synchronize()
    return specs, list(host_inputs(config)), banks


def _ns_slots(config, bi, spec):
    want = SAMPLES[config]["ns"]
    sel = want if want is None else want.get(bi, [])
    if sel is None:
        return list(spec.live_slots)
    if sel == "cover":
        return queue_cover(spec)
    return list(sel)


@pytest.mark.parametrize("config", [0, 1, 2, 3, 4, 5, 6, 7])
def test_bank_step_matches_oracle(config):
    say(f"bank step config {config}")
    api.mb_device_fault(clear=True)
    specs, host, banks = _run(config)
    torch.cuda.synchronize()
    assert not api.mb_device_fault(), "a persistent Newton-Schulz launch gave up a dependency wait"
    samp = SAMPLES[config]
    for bi, (spec, h, b) in enumerate(zip(specs, host, banks)):
        elem = list(range(spec.batch)) if samp["elem"] is None else samp["elem"][bi]
        storage = oracle.F32 if spec.grad_dtype == "f32" else oracle.BF16
        sc = oracle.step_scalars(0.02, 0.01, 0.95, spec.rows, spec.cols)
        g = vals(h["grad"][elem])
        m = vals(h["momentum"][elem])
        want_buf, want_u = oracle.momentum_nesterov(g, m, sc.mu, sc.nu, storage)
        got_buf = (b.momentum.float().cpu().numpy()[elem].astype(np.float64) if storage == oracle.F32
                   else vals(bits(b.momentum)[elem]))
        np.testing.assert_array_equal(got_buf, want_buf, err_msg=f"{spec.name} momentum")
        u_gpu = bits(b.u_out)
        np.testing.assert_array_equal(vals(u_gpu[elem]), want_u, err_msg=f"{spec.name} u")
        v_gpu = bits(b.v_out)
        # apply on the GPU's v: bit-exact
        want_hi, want_lo = oracle.mp_apply_update(h["w_hi"][elem], h["w_lo"][elem], vals(v_gpu[elem]), sc.eta,
                                                  sc.decay)
        np.testing.assert_array_equal(bits(b.w_hi)[elem], want_hi, err_msg=f"{spec.name} w_hi")
        np.testing.assert_array_equal(bits(b.w_lo)[elem], want_lo, err_msg=f"{spec.name} w_lo")
        # dead slots stay exactly zero everywhere
        for s in spec.dead_slots:
            assert np.all(bits(b.momentum)[s] == 0) if storage == oracle.BF16 else np.all(
                b.momentum[s].cpu().numpy() == 0)
            assert np.all(v_gpu[s] == 0) and np.all(u_gpu[s] == 0), f"{spec.name} dead slot {s}"
            assert np.all(bits(b.w_hi)[s] == 0) and np.all(bits(b.w_lo)[s] == 0)
        # Newton-Schulz on the GPU's u, slot by slot
        ns_slots = _ns_slots(config, bi, spec)
        if ns_slots:
            want_v = oracle.newton_schulz(vals(u_gpu[ns_slots]))
            err = rel_fro(vals(v_gpu[ns_slots]), want_v)
            say(f"  {spec.name} NS rel err on {len(ns_slots)} slots: max {err.max():.5f} (slot "
                f"{ns_slots[int(np.argmax(err))]}), min {err.min():.5f}")
            assert np.all(err <= NS_TOL), dict(zip(ns_slots, err))
            # end to end on those slots: |w_gpu - w_or| <= 1 ulp + eta |v_gpu - v_or|
            v_or = oracle.round_to_bf16(want_v)
            or_hi, or_lo = oracle.mp_apply_update(h["w_hi"][ns_slots], h["w_lo"][ns_slots], v_or, sc.eta, sc.decay)
            w_or = oracle.recombine(or_hi, or_lo).view(np.float32).astype(np.float64)
            w_gp = oracle.recombine(bits(b.w_hi)[ns_slots], bits(b.w_lo)[ns_slots]).view(np.float32).astype(np.float64)
            # each side rounds t - eta*v once, to half an ulp at its own magnitude
            half_ulps = 0.5 * (np.abs(np.spacing(w_or.astype(np.float32))).astype(np.float64) +
                               np.abs(np.spacing(w_gp.astype(np.float32))).astype(np.float64))
            bound = half_ulps + sc.eta * np.abs(vals(v_gpu[ns_slots]) - v_or)
            ratio = np.abs(w_gp - w_or) / bound
            say(f"  {spec.name} end-to-end |dw| / bound max {ratio.max():.4f}")
            assert np.all(np.abs(w_gp - w_or) <= bound)
    _check_paths_bitwise(config, banks)


def _check_paths_bitwise(config, banks0):
    """Every slot of every bank that the persistent launch runs gives the bits of one launch per
    contraction (same tile code, same k order), also where one launch carries several banks: a mistake in
    the launch's slot or bank decode, or in one XCD queue, shows in any slot it touches."""
    first = [(bits(b.v_out), bits(b.w_hi), bits(b.w_lo)) for b in banks0]
    prev = api.mb_ns_set_path(1)
    try:
        api.mb_device_fault(clear=True)
        _, _, banks1 = _run(config)
        assert not api.mb_device_fault()
        second = [(bits(b.v_out), bits(b.w_hi), bits(b.w_lo)) for b in banks1]
    finally:
        api.mb_ns_set_path(prev)
    checked = 0
    for spec, a, b in zip(WORKLOADS[config], first, second):
        if spec.rows % 128 or spec.cols % 128:
            continue                      # small and ragged slots take other kernels on the two paths
        for name, x, y in zip(("v", "w_hi", "w_lo"), a, b):
            bad = np.nonzero(np.any(x != y, axis=(1, 2)))[0]
            assert bad.size == 0, f"{spec.name} {name} differs from one launch per contraction on slots {bad.tolist()}"
        checked += 1
    assert checked > 0
    say(f"  {checked} persistent banks bit-identical to one launch per contraction on every slot")


def test_slot_scalar_table_matches_oracle():
    """Workload 3 (attention, MLP and both gate banks) with a per-slot table whose momentum, decay and
    learning rate differ from slot to slot: momentum and u bit-exact against the oracle with each slot's
    own scalars, the apply bit-exact on the GPU's v, Newton-Schulz within the tolerance on sampled slots."""
    say("bank step with a per-slot scalar table")
    config = 3
    specs, host = WORKLOADS[config], host_inputs(config)
    banks = _upload(config)
    table = api.slot_scalars_table(banks)
    rng = np.random.default_rng(123)
    mu = rng.uniform(0.8, 0.99, table.shape[0])
    table[:, 0] = mu.astype(np.float32)
    table[:, 1] = (1.0 - mu).astype(np.float32)
    table[:, 2] = rng.uniform(0.99, 1.0, table.shape[0]).astype(np.float32)
    table[:, 3] = (table[:, 3] * rng.uniform(0.5, 2.0, table.shape[0])).astype(np.float32)
    api.muon_bank_step(banks, api.with_slot_scalars(None, torch.from_numpy(table).cuda()))
    torch.cuda.synchronize()
    row = 0
    for spec, h, b in zip(specs, host, banks):
        tab = table[row:row + spec.batch].astype(np.float64)
        row += spec.batch
        mu_s, nu_s, d_s, eta_s = (tab[:, k][:, None, None] for k in range(4))
        want_buf, want_u = oracle.momentum_nesterov(vals(h["grad"]), vals(h["momentum"]), mu_s, nu_s, oracle.BF16)
        np.testing.assert_array_equal(vals(bits(b.momentum)), want_buf, err_msg=f"{spec.name} momentum")
        u = bits(b.u_out)
        np.testing.assert_array_equal(vals(u), want_u, err_msg=f"{spec.name} u")
        v = bits(b.v_out)
        hi, lo = oracle.mp_apply_update(h["w_hi"], h["w_lo"], vals(v), eta_s, d_s)
        np.testing.assert_array_equal(bits(b.w_hi), hi, err_msg=f"{spec.name} w_hi")
        np.testing.assert_array_equal(bits(b.w_lo), lo, err_msg=f"{spec.name} w_lo")
        live = list(spec.live_slots)
        ns = live[:2] + live[-1:]
        err = rel_fro(vals(v[ns]), oracle.newton_schulz(vals(u[ns])))
        assert np.all(err <= NS_TOL), err


def test_124m_step_is_five_launches():
    """The 124M model's whole step (attention, MLP and two gate banks) enqueues five kernels: momentum of
    every bank, their scales, the persistent Newton-Schulz launch, the gates' Newton-Schulz, every apply."""
    say("launch count")
    banks = _upload(3)
    ws = torch.empty(api.mb_step_workspace_bytes(banks), dtype=torch.uint8, device="cuda")
    api.muon_bank_step(banks, workspace=ws)
    torch.cuda.synchronize()
    api.mb_timing_enable(True)
    api.mb_timing_read()
    api.muon_bank_step(banks, workspace=ws)
    torch.cuda.synchronize()
    counts = {k: n for k, (n, _) in api.mb_timing_read().items()}
    api.mb_timing_enable(False)
    say(f"  launches {counts}")
    assert counts == {"momentum": 1, "ns_scale": 1, "ns_persist": 1, "ns_small": 1, "apply": 1}


def test_bank_step_is_deterministic():
    say("bank step determinism")
    outs = []
    for _ in range(2):
        specs, host, banks = _run(1)
        outs.append([(bits(b.w_hi), bits(b.w_lo), bits(b.v_out)) for b in banks])
    for a, b in zip(outs[0], outs[1]):
        for x, y in zip(a, b):
            np.testing.assert_array_equal(x, y)


def test_per_slot_lr_and_multipliers():
    say("bank step per-slot lr")
    h = make_bank(1, 0, slots=list(range(6)))
    per = np.array([1.0, 0.5, 2.0, 1.0, 0.25, 3.0], dtype=np.float32)
    b = api.Bank(grad=to_dev(h["grad"], True), momentum=to_dev(h["momentum"], True), w_hi=to_dev(h["w_hi"]),
                 w_lo=to_dev(h["w_lo"]), lr_mul=1.5, wd_mul=2.0, lr_mul_per_slot=to_dev(per))
    b.v_out = torch.empty(h["w_hi"].shape, dtype=torch.int16, device="cuda")
    hp = api.make_hparams(lr=0.05, weight_decay=0.1, momentum=0.9)
    api.muon_bank_step([b], hp)
    torch.cuda.synchronize()
    sc = oracle.step_scalars(0.05, 0.1, 0.9, 768, 768, lr_mul=1.5, wd_mul=2.0)
    eta = oracle.round_to_f32(sc.eta * per.astype(np.float64))[:, None, None]
    v = vals(bits(b.v_out))
    want_hi, want_lo = oracle.mp_apply_update(h["w_hi"], h["w_lo"], v, eta, sc.decay)
    np.testing.assert_array_equal(bits(b.w_hi), want_hi)
    np.testing.assert_array_equal(bits(b.w_lo), want_lo)
    want_buf, _ = oracle.momentum_nesterov(vals(h["grad"]), vals(h["momentum"]), sc.mu, sc.nu, oracle.BF16)
    np.testing.assert_array_equal(vals(bits(b.momentum)), want_buf)


def _fresh_bank(config, index):
    h = make_bank(config, index)
    bf = WORKLOADS[config][index].grad_dtype == "bf16"
    b = api.Bank(grad=to_dev(h["grad"], bf), momentum=to_dev(h["momentum"], bf), w_hi=to_dev(h["w_hi"]),
                 w_lo=to_dev(h["w_lo"]))
    b.v_out = torch.empty(h["w_hi"].shape, dtype=torch.int16, device="cuda")
    return b


def test_steps_on_two_streams_at_once_match_one_after_the_other():
    """Two banks stepped concurrently on two streams (default priority), each with its own workspace,
    give the bits of the same steps run one after the other on the null stream: the persistent
    launches share no state, and each one's tasks wait only for tasks of the same launch."""
    say("two streams")
    seq = [_fresh_bank(1, 0), _fresh_bank(2, 0)]
    for b in seq:
        api.muon_bank_step([b])
    torch.cuda.synchronize()
    con = [_fresh_bank(1, 0), _fresh_bank(2, 0)]
    wss = [torch.empty(api.mb_step_workspace_bytes([b]), dtype=torch.uint8, device="cuda") for b in con]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for b, ws, st in zip(con, wss, streams):
        api.muon_bank_step([b], workspace=ws, stream=st)
    torch.cuda.synchronize()
    assert not api.mb_device_fault(), "a persistent Newton-Schulz launch gave up a dependency wait"
    for a, b in zip(seq, con):
        for x, y in ((a.w_hi, b.w_hi), (a.w_lo, b.w_lo), (a.v_out, b.v_out), (a.momentum, b.momentum)):
            np.testing.assert_array_equal(bits(x), bits(y))
