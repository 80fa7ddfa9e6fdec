"""The C ABI without a GPU: symbols, defaults, workspace queries and every
validation error path (all of which return before anything is launched)."""

import ctypes
import json
import math
import os
import re

import pytest

from newton_schulz_bank_amd import api
from tests.conftest import GOLDEN, ROOT

HEADER = os.path.join(ROOT, "include", "muonbank.h")

OK, NULL, SHAPE, DTYPE, ALIGN, WORKSPACE, ALIAS, VALUE = 0, 1, 2, 3, 4, 5, 6, 7


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*[A-Za-z_][\w\s\*]*?\b(\w+)\s*\(", text, flags=re.M)) - {"if"})


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(api.LIB_PATH):
        from newton_schulz_bank_amd import build
        build.build()
    return api.lib()


def test_every_declared_symbol_is_exported(L):
    names = header_functions()
    assert set(names) == set(api.EXPORTED), names
    for n in names:
        assert hasattr(L, n), n


def test_default_hparams_are_the_pages_values(L):
    coef = json.load(open(os.path.join(GOLDEN, "ns_coefficients.json")))
    dflt = json.load(open(os.path.join(GOLDEN, "muon_defaults.json")))
    hp = api.default_hparams()
    assert (hp.a, hp.b, hp.c, hp.ns_steps) == (coef["a"], coef["b"], coef["c"], coef["steps"])
    assert (hp.lr, hp.weight_decay, hp.momentum) == (dflt["lr"], dflt["weight_decay"], dflt["momentum"])
    assert hp.eps == 1e-7
    assert L.mb_version().decode().startswith("muonbank")


def test_status_strings(L):
    assert L.mb_status_string(0) == b"ok"
    assert L.mb_status_string(5) == b"workspace too small"
    assert L.mb_status_string(99) == b"unknown status"


def test_workspace_queries(L):
    w1 = L.mb_ns_workspace_bytes(40, 768, 768)
    assert w1 >= 3 * 40 * 768 * 768 * 2 + 2 * 40 * 768 * 768 * 2
    assert L.mb_ns_workspace_bytes(24, 3072, 768) > w1
    assert L.mb_ns_workspace_bytes(0, 768, 768) == 0
    assert L.mb_ns_workspace_bytes(1, -1, 768) == 0
    b = api.mb_bank(40, 768, 768, api.MB_BF16, 1.0, 1.0, 0x10000, 0x20000, 0x30000, 0x40000, None, None, None)
    arr = (api.mb_bank * 2)(b, b)
    # per bank the Newton-Schulz workspace, plus one small block of queue heads and slot counters for
    # the persistent launch over all banks
    assert 2 * w1 < L.mb_step_workspace_bytes(arr, 2) <= 2 * w1 + 4096
    assert w1 < L.mb_step_workspace_bytes(arr, 1) <= w1 + 4096
    assert L.mb_step_workspace_bytes(arr, 0) == 0


def _bank(batch=4, rows=64, cols=64, dtype=api.MB_BF16, base=1 << 32, **over):
    n = batch * rows * cols
    es = 4 if dtype == api.MB_F32 else 2
    span = (n * max(es, 2) + 4095) // 4096 * 4096
    fields = dict(batch=batch, rows=rows, cols=cols, grad_dtype=dtype, lr_mul=1.0, wd_mul=1.0,
                  grad=base, momentum=base + span, w_hi=base + 2 * span, w_lo=base + 3 * span,
                  lr_mul_per_slot=None, v_out=None, u_out=None)
    fields.update(over)
    b = api.mb_bank()
    for k, v in fields.items():
        setattr(b, k, v)
    return b, base + 8 * span


def _step(L, banks, ws, ws_bytes, hp=None):
    arr = (api.mb_bank * len(banks))(*banks)
    return L.muon_bank_step(arr, len(banks), ctypes.byref(hp) if hp is not None else None, ws, ws_bytes, None)


def test_step_validation_errors(L):
    good, ws = _bank()
    need = L.mb_step_workspace_bytes((api.mb_bank * 1)(good), 1)
    assert _step(L, [_bank(grad=None)[0]], ws, need) == NULL
    assert L.muon_bank_step(None, 1, None, ws, need, None) == NULL
    assert _step(L, [_bank(rows=0)[0]], ws, need) == SHAPE
    assert _step(L, [_bank(batch=70000)[0]], ws, need) == SHAPE
    assert _step(L, [_bank(dtype=7)[0]], ws, need) == DTYPE
    assert _step(L, [_bank(grad=(1 << 32) + 2)[0]], ws, need) == ALIGN
    assert _step(L, [_bank(v_out=(1 << 40) + 8)[0]], ws, need) == ALIGN
    assert _step(L, [_bank(lr_mul_per_slot=(1 << 40) + 2)[0]], ws, need) == ALIGN
    assert _step(L, [good], ws, need - 1) == WORKSPACE
    assert _step(L, [good], None, need) == WORKSPACE
    # buffers overlapping each other, the workspace, or another bank
    assert _step(L, [_bank(momentum=good.grad + 1024)[0]], ws, need) == ALIAS
    assert _step(L, [good], good.w_lo, need) == ALIAS
    two = (api.mb_bank * 2)(good, good)
    assert L.muon_bank_step(two, 2, None, ws, 2 * need, None) == ALIAS
    hp = api.default_hparams()
    hp.ns_steps = 0
    assert _step(L, [good], ws, need, hp) == VALUE
    hp = api.default_hparams()
    hp.lr = math.nan
    assert _step(L, [good], ws, need, hp) == VALUE
    assert _step(L, [_bank(lr_mul=math.inf)[0]], ws, need) == VALUE
    hp = api.make_hparams(schedule=[(3.4445, -4.775, 2.0315), (1.0, math.nan, 0.0)])
    assert _step(L, [good], ws, need, hp) == VALUE
    assert b"schedule" in L.mb_last_error()
    assert len(L.mb_last_error()) > 0


def test_stage_entry_point_validation_errors(L):
    p = 1 << 36
    # momentum
    assert L.muon_momentum_update(None, p, p + (1 << 30), 1, 8, 8, 1, 0.95, 0.05, None) == NULL
    assert L.muon_momentum_update(p, p + (1 << 30), p + (2 << 30), 1, 8, 8, 9, 0.95, 0.05, None) == DTYPE
    assert L.muon_momentum_update(p, p + (1 << 30), p + (2 << 30), 0, 8, 8, 1, 0.95, 0.05, None) == SHAPE
    assert L.muon_momentum_update(p + 4, p + (1 << 30), p + (2 << 30), 1, 8, 8, 1, 0.95, 0.05, None) == ALIGN
    assert L.muon_momentum_update(p, p + 64, p + (2 << 30), 1, 8, 8, 1, 0.95, 0.05, None) == ALIAS
    assert L.muon_momentum_update(p, p + (1 << 30), p + (2 << 30), 1, 8, 8, 1, math.nan, 0.05, None) == VALUE
    # Newton-Schulz
    need = L.mb_ns_workspace_bytes(2, 64, 64)
    ws = p + (4 << 30)
    assert L.ns_orthogonalize_batched(None, p, 2, 64, 64, 5, 3.4445, -4.775, 2.0315, 1e-7, ws, need, None) == NULL
    assert L.ns_orthogonalize_batched(p, p + (1 << 30), 2, 64, 0, 5, 3.4445, -4.775, 2.0315, 1e-7, ws, need, None) == SHAPE
    assert L.ns_orthogonalize_batched(p, p + (1 << 30), 2, 64, 64, 0, 3.4445, -4.775, 2.0315, 1e-7, ws, need, None) == VALUE
    assert L.ns_orthogonalize_batched(p, p + (1 << 30), 2, 64, 64, 5, math.inf, -4.775, 2.0315, 1e-7, ws, need, None) == VALUE
    assert L.ns_orthogonalize_batched(p, p + (1 << 30), 2, 64, 64, 5, 3.4445, -4.775, 2.0315, 1e-7, ws, need - 1, None) == WORKSPACE
    assert L.ns_orthogonalize_batched(p, p + 16, 2, 64, 64, 5, 3.4445, -4.775, 2.0315, 1e-7, ws, need, None) == ALIAS
    assert L.ns_orthogonalize_batched(p, p + (1 << 30), 2, 64, 64, 5, 3.4445, -4.775, 2.0315, 1e-7, p + 256, need, None) == ALIAS
    assert L.ns_orthogonalize_batched(p + 2, p + (1 << 30), 2, 64, 64, 5, 3.4445, -4.775, 2.0315, 1e-7, ws, need, None) == ALIGN
    # Newton-Schulz with per-round coefficients
    sched = (ctypes.c_double * 6)(3.4445, -4.775, 2.0315, 3.0, -3.2, 1.2)
    bad = (ctypes.c_double * 6)(3.4445, -4.775, 2.0315, 3.0, math.inf, 1.2)
    assert L.ns_orthogonalize_batched_sched(p, p + (1 << 30), 2, 64, 64, 2, None, 1e-7, ws, need, None) == NULL
    assert L.ns_orthogonalize_batched_sched(p, p + (1 << 30), 2, 64, 64, 2, bad, 1e-7, ws, need, None) == VALUE
    assert L.ns_orthogonalize_batched_sched(p, p + (1 << 30), 2, 64, 64, 0, sched, 1e-7, ws, need, None) == VALUE
    assert L.ns_orthogonalize_batched_sched(p, p + (1 << 30), 2, 64, 64, 65, sched, 1e-7, ws, need, None) == VALUE
    assert L.ns_orthogonalize_batched_sched(p, p + (1 << 30), 2, 64, 64, 2, sched, 1e-7, ws, need - 1, None) == WORKSPACE
    # transposes
    assert L.transpose_copy(None, p, 8, 8, 2, None) == NULL
    assert L.transpose_copy(p, p + (1 << 30), 8, 0, 2, None) == SHAPE
    assert L.transpose_copy(p, p + (1 << 30), 8, 8, 3, None) == DTYPE
    assert L.transpose_copy(p + 1, p + (1 << 30), 8, 8, 2, None) == ALIGN
    assert L.transpose_copy(p, p + 64, 8, 8, 2, None) == ALIAS
    assert L.transpose_add(p, p + (1 << 30), 8, 8, 5, None) == DTYPE
    assert L.transpose_add(p + 2, p + (1 << 30), 8, 8, 0, None) == ALIGN
    # apply
    assert L.mp_apply_update(None, p, p, 1, 64, 0.02, 0.9998, None, None) == NULL
    assert L.mp_apply_update(p, p + (1 << 30), p + (2 << 30), 1, 0, 0.02, 0.9998, None, None) == SHAPE
    assert L.mp_apply_update(p, p + (1 << 30), p + (2 << 30), 1, 64, math.nan, 0.9998, None, None) == VALUE
    assert L.mp_apply_update(p, p + 32, p + (2 << 30), 1, 64, 0.02, 0.9998, None, None) == ALIAS
    assert L.mp_apply_update(p, p + (1 << 30), p + (2 << 30), 1, 64, 0.02, 0.9998, p + (3 << 30) + 2, None) == ALIGN


def test_binding_fails_loudly_without_the_library(monkeypatch):
    monkeypatch.setattr(api, "LIB_PATH", "/nonexistent/libmuonbank.so")
    monkeypatch.setattr(api, "_lib", None)
    with pytest.raises(RuntimeError, match="missing"):
        api.lib()


def test_device_fault_without_a_device_is_an_error(L):
    """With no GPU the flag cannot be read: -1 and a detail string, never a made-up 0 or 1; the binding
    raises."""
    try:
        import torch
        if torch.cuda.is_available():
            pytest.skip("a GPU is present: the flag is read for real by the GPU tests")
    except ImportError:
        pass
    assert L.mb_device_fault(0) == -1
    assert "mb_device_fault" in L.mb_last_error().decode()
    with pytest.raises(api.MuonBankError):
        api.mb_device_fault()


class _NoCalls:
    """Stands in for the library: any attribute access means a call was about to be made."""

    def __getattr__(self, name):
        raise AssertionError(f"the binding reached the library ({name}) with an invalid argument")


def test_binding_rejects_a_bad_per_slot_vector_before_any_call(monkeypatch):
    """mp_apply_update and Bank check lr_mul_per_slot (float32, one element per slot) before anything
    reaches the C ABI, which would read `batch` floats from the pointer.  Run with host tensors: the
    device-residency half of the check is relaxed so that the size and dtype halves are what reject."""
    import torch

    def host_dense(t, name, elem_size=2):
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        sizes = elem_size if isinstance(elem_size, tuple) else (elem_size,)
        if t.element_size() not in sizes:
            raise ValueError(f"{name} must have {sizes}-byte elements")

    monkeypatch.setattr(api, "_dense", host_dense)
    monkeypatch.setattr(api, "lib", lambda: _NoCalls())
    w_hi = torch.zeros((4, 8, 8), dtype=torch.int16)
    w_lo = torch.zeros_like(w_hi)
    v = torch.zeros_like(w_hi)
    with pytest.raises(ValueError, match="4 elements"):
        api.mp_apply_update(w_hi, w_lo, v, 0.02, 0.9998, lr_mul_per_slot=torch.ones(3, dtype=torch.float32))
    with pytest.raises(ValueError, match="float32"):
        api.mp_apply_update(w_hi, w_lo, v, 0.02, 0.9998, lr_mul_per_slot=torch.ones(4, dtype=torch.int32))
    g = torch.zeros((4, 8, 8), dtype=torch.bfloat16)
    bank = api.Bank(grad=g, momentum=g.clone(), w_hi=w_hi, w_lo=w_lo, lr_mul_per_slot=torch.ones(5))
    with pytest.raises(ValueError, match="4 elements"):
        bank.to_c()


def test_noalloc_rejects_oversized_shapes_before_touching_the_device(L):
    """The size check of the allocation-free entry point comes before any device call, so it answers
    without a GPU; shapes within the limit would need the device and are left to the GPU tests."""
    p = 1 << 36
    big = (200, 768, 768)
    assert L.mb_ns_workspace_bytes(*big) > (256 << 20)
    assert L.ns_orthogonalize_batched_noalloc(p, p + (1 << 30), *big, 5, 3.4445, -4.775, 2.0315, 1e-7, None) == WORKSPACE
    assert b"static scratch" in L.mb_last_error()
    assert L.ns_orthogonalize_batched_noalloc(p, p + (1 << 30), 0, 768, 768, 5, 3.4445, -4.775, 2.0315, 1e-7, None) == SHAPE


def test_slot_scalars_fill_is_the_call_scalars(L):
    """The host table holds, per slot in bank order, the float32 (mu, nu, decay, eta) the step derives
    from the hyper-parameters and each bank's multipliers; the oracle's step_scalars gives the same
    values."""
    import numpy as np
    import oracle
    b1, _ = _bank(batch=3, rows=64, cols=32)
    b2, _ = _bank(batch=2, rows=16, cols=64, base=1 << 40)
    b2.lr_mul, b2.wd_mul = 1.5, 0.5
    hp = api.make_hparams(lr=0.05, weight_decay=0.1, momentum=0.9)
    arr = (api.mb_bank * 2)(b1, b2)
    out = np.zeros((5, 4), dtype=np.float32)
    assert L.mb_slot_scalars_fill(arr, 2, ctypes.byref(hp), out.ctypes.data, out.size) == OK
    for rows, (r, c, lm, wm) in zip((range(0, 3), range(3, 5)), ((64, 32, 1.0, 1.0), (16, 64, 1.5, 0.5))):
        sc = oracle.step_scalars(0.05, 0.1, 0.9, r, c, lr_mul=lm, wd_mul=wm)
        for i in rows:
            assert tuple(out[i].astype(np.float64)) == (sc.mu, sc.nu, sc.decay, sc.eta)
    assert L.mb_slot_scalars_fill(arr, 2, ctypes.byref(hp), out.ctypes.data, out.size - 1) == WORKSPACE
    b3, _ = _bank(lr_mul_per_slot=1 << 44)
    assert L.mb_slot_scalars_fill((api.mb_bank * 1)(b3), 1, None, out.ctypes.data, out.size) == VALUE
    assert L.mb_slot_scalars_fill(None, 1, None, out.ctypes.data, out.size) == NULL


def test_step_with_slot_scalars_validation(L):
    good, ws = _bank()
    need = L.mb_step_workspace_bytes((api.mb_bank * 1)(good), 1)
    hp = api.default_hparams()
    hp.slot_scalars = (1 << 46) + 8
    assert _step(L, [good], ws, need, hp) == ALIGN
    hp.slot_scalars = good.grad + 64
    assert _step(L, [good], ws, need, hp) == ALIAS
    hp.slot_scalars = 1 << 46
    assert _step(L, [_bank(lr_mul_per_slot=1 << 44)[0]], ws, need, hp) == VALUE
    assert b"lr_mul_per_slot" in L.mb_last_error()


def test_persist_fault_hook_validation(L):
    """The failure-path test hook rejects a negative wait cap and extra queues outside 0..8 (host only)."""
    assert L.mb_test_persist_faults(-1, 0) == VALUE
    assert L.mb_test_persist_faults(0, 9) == VALUE
    assert L.mb_test_persist_faults(0, -1) == VALUE
    assert L.mb_test_persist_faults(0, 0) == 0
