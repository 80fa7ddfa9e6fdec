"""The tied-embedding transposes on the GPU against the oracle, bit for bit.

transpose_copy is a bit copy and transpose_add rounds the exact sum once, so
every compared element must be identical.  The full LM-head shape (768, 50304)
and its reverse run through the tiled kernels, with the copy compared on
every element and the add on sampled destination rows.  Ragged shapes and
unaligned buffers run through the element-wise kernel.
"""

import sys

import numpy as np
import pytest
import torch

import oracle
from newton_schulz_bank_amd import api

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _rand(rng, shape, kind):
    if kind == "bf16":
        return oracle.f64_to_bf16_bits(oracle.round_to_bf16(rng.normal(0, 0.02, shape)))
    if kind == "f32":
        return rng.normal(0, 0.02, shape).astype(np.float32)
    return rng.integers(0, 65536, shape).astype(np.uint16)


def _dev(a, kind):
    if a.dtype == np.uint16:
        t = torch.from_numpy(a.view(np.int16)).cuda()
        return t.view(torch.bfloat16) if kind == "bf16" else t
    return torch.from_numpy(a).cuda()


def _host(t):
    if t.dtype in (torch.bfloat16, torch.int16):
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


SHAPES = [(768, 50304), (50304, 768), (64, 64), (128, 192), (100, 260), (37, 5), (1, 12), (65, 129), (8, 1000)]


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("kind", ["bits16", "f32"])
def test_transpose_copy(shape, kind):
    say(f"transpose_copy {shape} {kind}")
    rng = np.random.default_rng(sum(shape))
    src = _rand(rng, shape, kind)
    ds = _dev(src, kind)
    dd = torch.empty((shape[1], shape[0]), dtype=ds.dtype, device="cuda")
    api.transpose_copy(dd, ds)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(_host(dd), oracle.transpose_copy(src))


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("kind", ["bf16", "f32"])
def test_transpose_add(shape, kind):
    say(f"transpose_add {shape} {kind}")
    rng = np.random.default_rng(7 + sum(shape))
    src = _rand(rng, shape, kind)
    dst = _rand(rng, (shape[1], shape[0]), kind)
    dd = _dev(dst, kind)
    api.transpose_add(dd, _dev(src, kind))
    torch.cuda.synchronize()
    got = _host(dd)
    fmt = oracle.BF16 if kind == "bf16" else oracle.F32
    if shape[0] * shape[1] > 1 << 20:
        rows = np.sort(rng.choice(shape[1], 256, replace=False))      # sampled dst rows = src columns
        want = oracle.transpose_add(dst[rows], np.ascontiguousarray(src[:, rows]), fmt)
        np.testing.assert_array_equal(got[rows], want)
    else:
        np.testing.assert_array_equal(got, oracle.transpose_add(dst, src, fmt))


def test_unaligned_buffers_take_the_elementwise_kernel():
    say("transpose unaligned")
    rng = np.random.default_rng(11)
    src = _rand(rng, (96, 64), "bits16")
    base = torch.from_numpy(np.concatenate([[0], src.ravel()]).astype(np.uint16).view(np.int16)).cuda()
    ds = base[1:].view(96, 64)                     # 2 bytes past a 16-byte boundary
    out = torch.zeros(64 * 96 + 1, dtype=torch.int16, device="cuda")
    dd = out[1:].view(64, 96)
    api.transpose_copy(dd, ds)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(_host(dd), oracle.transpose_copy(src))
    assert int(out[0]) == 0
