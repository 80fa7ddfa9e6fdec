"""muon_bank_step captured in a HIP graph (torch.cuda.graph) and replayed.

The library enqueues kernels and (for one-round calls) a device-to-device copy
only: no memset, no allocation, no synchronisation, so a whole step can be
captured once and replayed.  Every replay is compared bit for bit with the same
step run eagerly from the same inputs, with eager work and synchronisations
between the replays.
"""

import sys

import numpy as np
import pytest
import torch

from newton_schulz_bank_amd import api
from newton_schulz_bank_amd.workloads import WORKLOADS, make_bank
from tests.gpu_util import bits, to_dev

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _banks(config):
    out = []
    for i, spec in enumerate(WORKLOADS[config]):
        h = make_bank(config, i)
        bf = spec.grad_dtype == "bf16"
        out.append((h, bf))
    return out


def _upload(hosts):
    banks = []
    for h, bf in hosts:
        b = api.Bank(grad=to_dev(h["grad"], bf), momentum=to_dev(h["momentum"], bf), w_hi=to_dev(h["w_hi"]),
                     w_lo=to_dev(h["w_lo"]))
        b.v_out = torch.zeros(h["w_hi"].shape, dtype=torch.int16, device="cuda")
        banks.append(b)
    return banks


def _state(banks):
    return [(bits(b.momentum), bits(b.w_hi), bits(b.w_lo), bits(b.v_out)) for b in banks]


@pytest.mark.parametrize("config", [1, 3])
def test_graph_replays_match_eager_steps(config):
    say(f"graph capture, workload {config}")
    hosts = _banks(config)
    # eager reference: three consecutive steps from the pristine inputs
    eager = _upload(hosts)
    ws = torch.empty(api.mb_step_workspace_bytes(eager), dtype=torch.uint8, device="cuda")
    want = []
    for _ in range(3):
        api.muon_bank_step(eager, workspace=ws)
        torch.cuda.synchronize()
        want.append(_state(eager))
    # captured: one step, replayed three times on freshly uploaded inputs
    banks = _upload(hosts)
    ws2 = torch.empty_like(ws)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        # warm-up outside the capture on scratch copies (first-call set-up happens here)
        scratch = _upload(hosts)
        api.muon_bank_step(scratch, workspace=ws2)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        api.muon_bank_step(banks, workspace=ws2)
    for k in range(3):
        g.replay()
        torch.cuda.synchronize()
        got = _state(banks)
        for bi, (a, b) in enumerate(zip(got, want[k])):
            for name, x, y in zip(("momentum", "w_hi", "w_lo", "v"), a, b):
                np.testing.assert_array_equal(x, y, err_msg=f"replay {k} bank {bi} {name}")
        # eager work between replays
        junk = torch.randn(1 << 20, device="cuda").sum()
        torch.cuda.synchronize()
        assert torch.isfinite(junk)


def test_graph_replays_read_the_current_slot_scalars():
    """A step captured with a per-slot scalar table reads the table when it replays: between replays the
    table's device buffer is overwritten (an ordinary copy into the same memory, as a training loop
    uploads each step's momentum, decay and learning rates), and every replay equals the eager step
    taken with that replay's table."""
    say("graph capture with a per-slot scalar table")
    hosts = _banks(3)
    eager = _upload(hosts)
    base = api.slot_scalars_table(eager)
    rng = np.random.default_rng(77)
    tables = []
    for k in range(3):
        t = base.copy()
        mu = rng.uniform(0.85, 0.99, t.shape[0])
        t[:, 0] = mu.astype(np.float32)
        t[:, 1] = (1.0 - mu).astype(np.float32)
        t[:, 2] = rng.uniform(0.995, 1.0, t.shape[0]).astype(np.float32)
        t[:, 3] = (t[:, 3] * rng.uniform(0.5, 1.5, t.shape[0])).astype(np.float32)
        tables.append(t)
    ws = torch.empty(api.mb_step_workspace_bytes(eager), dtype=torch.uint8, device="cuda")
    dev_tab = torch.empty((base.shape[0], 4), dtype=torch.float32, device="cuda")
    hp = api.with_slot_scalars(None, dev_tab)
    want = []
    for t in tables:
        dev_tab.copy_(torch.from_numpy(t))
        api.muon_bank_step(eager, hp=hp, workspace=ws)
        torch.cuda.synchronize()
        want.append(_state(eager))
    banks = _upload(hosts)
    ws2 = torch.empty_like(ws)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        scratch = _upload(hosts)
        api.muon_bank_step(scratch, hp=hp, workspace=ws2)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        api.muon_bank_step(banks, hp=hp, workspace=ws2)
    for k, t in enumerate(tables):
        dev_tab.copy_(torch.from_numpy(t))
        g.replay()
        torch.cuda.synchronize()
        for bi, (a, b) in enumerate(zip(_state(banks), want[k])):
            for name, x, y in zip(("momentum", "w_hi", "w_lo", "v"), a, b):
                np.testing.assert_array_equal(x, y, err_msg=f"replay {k} bank {bi} {name}")
