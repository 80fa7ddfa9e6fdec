"""Failure paths of the persistent Newton-Schulz launch, forced from the host through the library's test hook
(mb_test_persist_faults), on the GPU: a dependency wait that gives up at a one-tick cap, and an XCD queue that no
workgroup serves (the end-of-launch drain check).  Both launches finish normally, and the fault flag reports
them.  With the hook reset, the same call is correct and clean again."""

import sys

import numpy as np
import pytest
import torch

from newton_schulz_bank_amd import api
from newton_schulz_bank_amd.workloads import random_bf16_matrices
from tests.gpu_util import bits, to_dev

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, file=sys.stderr, flush=True)


def _per_round(dx):
    prev = api.mb_ns_set_path(1)
    try:
        return bits(api.ns_orthogonalize_batched(dx))
    finally:
        api.mb_ns_set_path(prev)


def test_a_wait_at_its_cap_sets_the_fault_flag_and_the_launch_finishes():
    say("fault: wait cap of one tick, one 3072 x 768 slot")
    # one tall slot: every task sits on one XCD queue, and its polynomial tiles wait for a Gram of k = 3072
    x = random_bf16_matrices(41, 1, 3072, 768, scale=1e-3)
    dx = to_dev(x)
    ref = _per_round(dx)
    api.mb_device_fault(clear=True)
    try:
        api.mb_test_persist_faults(wait_cap_ticks=1)
        api.ns_orthogonalize_batched(dx)
        torch.cuda.synchronize()
        assert api.mb_device_fault(clear=True), "a one-tick wait cap did not report a fault"
    finally:
        api.mb_test_persist_faults(0, 0)
    got = bits(api.ns_orthogonalize_batched(dx))
    torch.cuda.synchronize()
    assert not api.mb_device_fault()
    np.testing.assert_array_equal(got, ref)


def test_an_unserved_queue_sets_the_fault_flag_and_the_served_slots_are_right():
    say("fault: one extra queue that no XCD serves, nine 256 x 256 slots")
    x = random_bf16_matrices(42, 9, 256, 256, scale=1e-3)
    dx = to_dev(x)
    ref = _per_round(dx)
    api.mb_device_fault(clear=True)
    try:
        api.mb_test_persist_faults(extra_queues=1)
        got = bits(api.ns_orthogonalize_batched(dx))
        torch.cuda.synchronize()
        assert api.mb_device_fault(clear=True), "a queue left undrained was not reported"
    finally:
        api.mb_test_persist_faults(0, 0)
    # slot g runs on queue g % 9: slot 8 sits on the unserved queue, slots 0..7 on the XCDs' own
    np.testing.assert_array_equal(got[:8], ref[:8])
    got = bits(api.ns_orthogonalize_batched(dx))
    torch.cuda.synchronize()
    assert not api.mb_device_fault()
    np.testing.assert_array_equal(got, ref)
