"""The step planner and the persistent launch's task lists, on the host (no GPU).

mb_step_plan plans a step exactly as muon_bank_step does and checks every persistent launch's task
lists with the kernel's own decode (every task of every slot listed once, on its slot's XCD queue,
after each task it waits for).  These tests run it on every workload, on several XCD counts and on
random mixes of banks."""

import ctypes
import os

import numpy as np
import pytest

from newton_schulz_bank_amd import api
from newton_schulz_bank_amd.workloads import WORKLOADS


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(api.LIB_PATH):
        from newton_schulz_bank_amd import build
        build.build()
    return api.lib()


def _banks(shapes):
    out = []
    base = 1 << 36
    for b, r, c in shapes:
        out.append(api.mb_bank(b, r, c, api.MB_BF16, 1.0, 1.0, base, base + 8, base + 16, base + 24, None, None, None))
        base += 1 << 32
    return (api.mb_bank * len(out))(*out), len(out)


def plan(L, shapes, xcds=8, hp=None, cus=None):
    arr, n = _banks(shapes)
    info = api.mb_step_plan_info()
    cus = 32 * xcds if cus is None else cus
    st = L.mb_step_plan(arr, n, ctypes.byref(hp) if hp is not None else None, cus, xcds, ctypes.byref(info))
    assert st == 0, L.mb_last_error().decode()
    return info


def shapes_of(config):
    return [(s.batch, s.rows, s.cols) for s in WORKLOADS[config]]


@pytest.mark.parametrize("config", sorted(WORKLOADS))
@pytest.mark.parametrize("xcds", [8, 1, 3, 6, 16])
def test_every_workload_plans_and_its_task_lists_check(L, config, xcds):
    plan(L, shapes_of(config), xcds)


def test_the_124m_step_is_five_launches(L):
    info = plan(L, shapes_of(3))
    assert (info.momentum, info.ns_scale, info.ns_persist, info.ns_small, info.ns_per_contraction, info.apply) == \
        (1, 1, 1, 1, 0, 1)
    assert info.total == 5 and info.copies == 0
    assert info.persist_tile[0] == 256


def test_tile_choices(L):
    # 350M banks: one launch of all three banks, 256-tiles
    info = plan(L, shapes_of(4))
    assert info.ns_persist == 1 and info.persist_tile[0] == 256 and info.total == 4
    # one GPU's share of the 124M banks: 8 slots, 128-tiles
    info = plan(L, shapes_of(5))
    assert info.ns_persist == 1 and info.persist_tile[0] == 128
    # four 256^2 slots (the fp32 workload): 128-tiles
    assert plan(L, shapes_of(0)).persist_tile[0] == 128


def test_per_contraction_path_and_unknown_layout(L):
    prev = api.mb_ns_set_path(1)
    try:
        info = plan(L, shapes_of(3))
    finally:
        api.mb_ns_set_path(prev)
    # every bank, gates included, takes three launches per round
    assert info.ns_persist == 0 and info.ns_small == 0 and info.ns_per_contraction == 4 * 3 * 5
    # a device whose XCD layout the persistent launch does not take
    info = plan(L, shapes_of(1), xcds=0)
    assert info.ns_persist == 0 and info.ns_per_contraction == 15


def test_random_bank_mixes(L):
    """Random launches of 1..8 banks of multiple-of-128 slots (wide, tall, square), 1..40 slots each, on
    1..16 queues: the task lists of every launch check."""
    rng = np.random.default_rng(2024)
    for _ in range(60):
        nb = int(rng.integers(1, 9))
        shapes = []
        for _ in range(nb):
            r, c = (int(rng.integers(1, 9)) * 128 for _ in range(2))
            shapes.append((int(rng.integers(1, 41)), r, c))
        steps = int(rng.integers(1, 7))
        plan(L, shapes, int(rng.integers(1, 17)), api.make_hparams(ns_steps=steps))


def test_more_banks_than_one_launch_holds(L):
    # 20 banks: two launches of each streaming kernel, three persistent launches of at most 8 banks
    info = plan(L, [(3, 256, 512)] * 20)
    assert info.momentum == 2 and info.apply == 2 and info.ns_scale == 2
    assert info.ns_persist == 3


# (tile, ring, workgroups, claim_early) of each workload's persistent launch on 256 CUs in 8 XCDs: the
# three-slot ring from 128 MiB of X (the 124M step's two big banks: 160 MB; the 350M banks: 708 MB), early
# claims where every queue holds two rounds of tasks per workgroup (not one slot per XCD: workloads 0, 5)
LAUNCHES = {0: (128, 2, 256, 0), 1: (256, 2, 256, 1), 2: (256, 2, 256, 1), 3: (256, 3, 256, 1),
            4: (256, 3, 256, 1), 5: (128, 2, 512, 0), 6: (256, 2, 256, 1), 7: (256, 3, 256, 1)}


@pytest.mark.parametrize("config", sorted(LAUNCHES))
def test_persistent_launch_choices(L, config):
    info = plan(L, shapes_of(config), 8, cus=256)
    assert info.ns_persist == 1
    got = (info.persist_tile[0], info.persist_ring[0], info.persist_workgroups[0], info.persist_claim_early[0])
    assert got == LAUNCHES[config], (config, got)


def test_ring_threshold_is_128_mib_of_x(L):
    """40 attention slots (47 MB of X) keep the two-stage ring; 112 of them (132 MB) too; 114 (134.5 MB) take
    the three-slot ring."""
    for batch, ring in ((40, 2), (112, 2), (114, 3)):
        info = plan(L, [(batch, 768, 768)], 8, cus=256)
        assert info.persist_ring[0] == ring, (batch, info.persist_ring[0])


def test_a_device_layout_the_launch_does_not_take(L):
    """With a CU count that is not a multiple of the XCD count the step plans no persistent launch: every
    contraction is its own launch."""
    info = plan(L, shapes_of(1), 8, cus=250)
    assert info.ns_persist == 0 and info.ns_per_contraction == 15
