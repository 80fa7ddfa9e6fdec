"""Host logic of bench.py that runs without a GPU: the one-GPU guard, the flop count it prices the
Newton-Schulz launch with, and the comparison of a GPU sample with the oracle in its CPU-baseline leg."""

import json
import os
import subprocess
import sys

import numpy as np
import pytest

import bench
import oracle
from newton_schulz_bank_amd.workloads import WORKLOADS, make_bank

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in json.loads(r.stdout.strip().splitlines()[-1])["error"]


@pytest.mark.parametrize("m,n", [(4, 6), (3, 8), (5, 5)])
def test_flop_count_matches_a_count_of_multiply_adds(m, n):
    """Count the multiply-adds of one round by enumerating them (a symmetric product counted on its
    upper triangle, as the kernels compute it): Gram X X^T (m x m from n-long dots), A A (m x m from
    m-long dots), B X (m x n from m-long dots)."""
    gram = sum(n for i in range(m) for j in range(i, m))
    poly = sum(m for i in range(m) for j in range(i, m))
    upd = sum(m for i in range(m) for j in range(n))
    per_round = 2 * (gram + poly + upd)
    f = bench.ns_flops_per_slot(m, n)
    assert sum(f.values()) == 5 * per_round
    assert sum(bench.ns_flops_per_slot(n, m).values()) == 5 * per_round   # tall = wide transposed
    # the dense-equivalent count takes every product in full: m x m from n (twice: X X^T is computed as
    # a whole), m x m from m, m x n from m
    dense = 2 * (m * m * n + m * m * m + m * n * m)
    assert bench.ns_dense_flops_per_slot(m, n) == bench.ns_dense_flops_per_slot(n, m) == 5 * dense


def _oracle_sample(spec, h, slot=None):
    """A GPU-shaped sample made by the oracle itself: it must pass the comparison."""
    slot = spec.live_slots[0] if slot is None else slot
    sl = lambda a: np.ascontiguousarray(a[slot:slot + 1])
    ref = oracle.muon_bank_step(oracle.bf16_bits_to_f64(sl(h["grad"])), oracle.bf16_bits_to_f64(sl(h["momentum"])),
                                sl(h["w_hi"]), sl(h["w_lo"]), oracle.BF16)
    return {"bank": spec.name, "slot": slot, "v": oracle.f64_to_bf16_bits(ref["v"]), "w_hi": ref["w_hi"],
            "w_lo": ref["w_lo"], "momentum": oracle.f64_to_bf16_bits(ref["momentum"])}


def test_sample_comparison_accepts_a_correct_step_and_rejects_a_flipped_bit():
    spec = WORKLOADS[1][0]                    # the attention bank; its slot 0 is live
    h = make_bank(1, 0, slots=[0])
    sample = _oracle_sample(spec, h)
    got = bench._sample_parity(oracle, spec, h, sample)
    assert got["apply_bit_exact"] and got["momentum_bit_exact"] and got["ns_rel_fro_err"] < 1e-2
    bad = dict(sample, w_lo=sample["w_lo"].copy())
    bad["w_lo"].flat[12345] ^= 1
    with pytest.raises(SystemExit):
        bench._sample_parity(oracle, spec, h, bad)


def test_parity_over_banks_checks_every_sample_and_reports_the_worst():
    """The bench samples the first and last live slot of every bank; each is compared with the oracle's
    step of that slot of its own bank, and one wrong bit anywhere fails the whole check."""
    specs = WORKLOADS[3][2:]                  # the two gate banks: (16, 1, 12) with one live slot, (16, 6, 12)
    hosts = [make_bank(3, 2 + i) for i in range(len(specs))]
    samples = [_oracle_sample(s, h, slot) for s, h in zip(specs, hosts)
               for slot in dict.fromkeys((s.live_slots[0], s.live_slots[-1]))]
    assert len(samples) == 3
    got = bench._parity(oracle, specs, hosts, samples)
    assert got["apply_bit_exact"] and got["momentum_bit_exact"]
    assert [(c["bank"], c["slot"]) for c in got["slots"]] == [(s["bank"], s["slot"]) for s in samples]
    assert got["ns_rel_fro_err_max"] == max(c["ns_rel_fro_err"] for c in got["slots"])
    bad = [dict(x) for x in samples]
    bad[-1]["momentum"] = bad[-1]["momentum"].copy()
    bad[-1]["momentum"].flat[3] ^= 1
    with pytest.raises(SystemExit):
        bench._parity(oracle, specs, hosts, bad)
