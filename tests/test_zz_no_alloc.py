"""The allocation-free Newton-Schulz entry point against the one with a caller's workspace.

ns_orthogonalize_batched_noalloc runs the same kernels as ns_orthogonalize_batched with its scratch in
the library's static device array, so on the same input the two give the same bits.  Two calls in a row,
the second on a smaller input, check that the array's leftovers from one call never reach the next.
"""

import numpy as np
import pytest
import torch

from newton_schulz_bank_amd import api
from newton_schulz_bank_amd.workloads import random_bf16_matrices
from tests.gpu_util import bits, to_dev

pytestmark = pytest.mark.gpu


def _both(x_bits, **kw):
    x = to_dev(x_bits)
    want = api.ns_orthogonalize_batched(x, **kw)
    y = torch.empty_like(x)
    torch.cuda.synchronize()
    api.ns_orthogonalize_batched_noalloc(x, y, **kw)
    torch.cuda.synchronize()
    return bits(want), bits(y)


def test_noalloc_matches_workspace_entry_point_on_two_calls():
    api.mb_device_fault(clear=True)
    # the attention bank (persistent launch, 256-tiles), then a smaller bank (128-tiles) in the same array
    for seed, shape in ((6100, (40, 768, 768)), (6101, (8, 256, 512))):
        print(f"noalloc {shape}", flush=True)
        x = random_bf16_matrices(seed, *shape, 1e-3)
        want, got = _both(x)
        np.testing.assert_array_equal(got, want, err_msg=str(shape))
        assert np.any(got != 0)
    assert not api.mb_device_fault()


def test_noalloc_in_place_ragged_and_single_round():
    for seed, shape, kw in ((6102, (3, 100, 260), {}), (6103, (4, 6, 12), {}), (6104, (2, 384, 128), {"steps": 1})):
        print(f"noalloc {shape} {kw}", flush=True)
        x = random_bf16_matrices(seed, *shape, 1e-3)
        want, got = _both(x, **kw)
        np.testing.assert_array_equal(got, want, err_msg=str(shape))
        # in place: y is x
        t = to_dev(x)
        api.ns_orthogonalize_batched_noalloc(t, t, **kw)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(bits(t), want, err_msg=f"{shape} in place")


def test_noalloc_rejects_a_shape_beyond_its_scratch():
    x = torch.empty((1, 8, 8), dtype=torch.int16, device="cuda")
    big = (200, 768, 768)
    assert api.mb_ns_workspace_bytes(*big) > 256 << 20
    st = api.lib().ns_orthogonalize_batched_noalloc(x.data_ptr(), x.data_ptr(), *big, 5, 3.4445, -4.775, 2.0315,
                                                    1e-7, None)
    assert st == 5 and b"static scratch" in api.lib().mb_last_error()
