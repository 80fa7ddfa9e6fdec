"""Python binding of libmuonbank.so: argument marshalling only.

Each function here has the name of the C entry point it calls (declared in
``include/muonbank.h``) and does nothing but check that tensors are dense
device tensors of the right element size, pass their pointers and the current
HIP stream, and turn a non-OK status into ``MuonBankError``.  All arithmetic
runs in the library's HIP kernels; there is no fallback.

bf16 bit tensors (weights ``w_hi``, Newton-Schulz input/output, u, v) may be
``torch.bfloat16``, ``torch.int16`` or ``torch.uint16`` -- only the 2-byte
storage matters.  The low mantissa ``w_lo`` is any 2-byte integer tensor.
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmuonbank.so")

MB_F32, MB_BF16 = 0, 1
_STATUS = {0: "MB_OK", 1: "MB_ERR_NULL", 2: "MB_ERR_SHAPE", 3: "MB_ERR_DTYPE", 4: "MB_ERR_ALIGN",
           5: "MB_ERR_WORKSPACE", 6: "MB_ERR_ALIAS", 7: "MB_ERR_VALUE", 8: "MB_ERR_HIP"}


vp_t = ctypes.c_void_p


class MuonBankError(RuntimeError):
    def __init__(self, status: int, message: str):
        self.status = status
        self.status_name = _STATUS.get(status, str(status))
        super().__init__(f"{self.status_name}: {message}")


class mb_hparams(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_double), ("weight_decay", ctypes.c_double), ("momentum", ctypes.c_double),
                ("ns_steps", ctypes.c_int32), ("a", ctypes.c_double), ("b", ctypes.c_double),
                ("c", ctypes.c_double), ("eps", ctypes.c_double), ("ns_schedule", ctypes.c_void_p),
                ("slot_scalars", ctypes.c_void_p)]


class mb_bank(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("rows", ctypes.c_int64), ("cols", ctypes.c_int64),
                ("grad_dtype", ctypes.c_int32), ("lr_mul", ctypes.c_double), ("wd_mul", ctypes.c_double),
                ("grad", ctypes.c_void_p), ("momentum", ctypes.c_void_p), ("w_hi", ctypes.c_void_p),
                ("w_lo", ctypes.c_void_p), ("lr_mul_per_slot", ctypes.c_void_p), ("v_out", ctypes.c_void_p),
                ("u_out", ctypes.c_void_p)]


class mb_step_plan_info(ctypes.Structure):
    _fields_ = [(k, ctypes.c_int32) for k in ("momentum", "ns_scale", "ns_persist", "ns_small", "ns_per_contraction",
                                              "apply", "copies", "total")] + \
               [(k, ctypes.c_int32 * 8) for k in ("persist_tile", "persist_ring", "persist_workgroups",
                                                  "persist_claim_early")]


class mb_kernel_time(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 48), ("launches", ctypes.c_int64), ("total_ms", ctypes.c_double)]


_lib = None

EXPORTED = ("mb_default_hparams", "mb_status_string", "mb_last_error", "mb_version", "mb_slot_scalars_fill",
            "mb_step_plan", "mb_step_workspace_bytes",
            "mb_ns_workspace_bytes", "muon_bank_step", "muon_momentum_update", "ns_orthogonalize_batched",
            "ns_orthogonalize_batched_sched", "ns_orthogonalize_batched_noalloc", "mp_apply_update", "transpose_copy", "transpose_add", "mb_ns_set_path", "mb_device_fault", "mb_test_persist_faults", "mb_timing_enable",
            "mb_timing_read")


def lib() -> ctypes.CDLL:
    """Load libmuonbank.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m newton_schulz_bank_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, f32, f64, sz = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float,
                                  ctypes.c_double, ctypes.c_size_t)
    sig = {
        "mb_default_hparams": (None, [ctypes.POINTER(mb_hparams)]),
        "mb_status_string": (ctypes.c_char_p, [i32]),
        "mb_last_error": (ctypes.c_char_p, []),
        "mb_version": (ctypes.c_char_p, []),
        "mb_step_workspace_bytes": (sz, [ctypes.POINTER(mb_bank), i32]),
        "mb_slot_scalars_fill": (i32, [ctypes.POINTER(mb_bank), i32, ctypes.POINTER(mb_hparams), vp, i64]),
        "mb_step_plan": (i32, [ctypes.POINTER(mb_bank), i32, ctypes.POINTER(mb_hparams), i32, i32,
                               ctypes.POINTER(mb_step_plan_info)]),
        "mb_ns_workspace_bytes": (sz, [i64, i64, i64]),
        "muon_bank_step": (i32, [ctypes.POINTER(mb_bank), i32, ctypes.POINTER(mb_hparams), vp, sz, vp]),
        "muon_momentum_update": (i32, [vp, vp, vp, i64, i64, i64, i32, f32, f32, vp]),
        "ns_orthogonalize_batched": (i32, [vp, vp, i64, i64, i64, i32, f64, f64, f64, f64, vp, sz, vp]),
        "ns_orthogonalize_batched_sched": (i32, [vp, vp, i64, i64, i64, i32, vp, f64, vp, sz, vp]),
        "ns_orthogonalize_batched_noalloc": (i32, [vp, vp, i64, i64, i64, i32, f64, f64, f64, f64, vp]),
        "mp_apply_update": (i32, [vp, vp, vp, i64, i64, f32, f32, vp, vp]),
        "mb_ns_set_path": (i32, [i32]),
        "mb_device_fault": (i32, [i32]),
        "mb_test_persist_faults": (i32, [i64, i32]),
        "transpose_copy": (i32, [vp, vp, i64, i64, i32, vp]),
        "transpose_add": (i32, [vp, vp, i64, i64, i32, vp]),
        "mb_timing_enable": (None, [i32]),
        "mb_timing_read": (i32, [ctypes.POINTER(mb_kernel_time), i32]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    _lib = L
    return L


def _check(status: int) -> None:
    if status != 0:
        raise MuonBankError(status, lib().mb_last_error().decode())


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _dense(t: torch.Tensor, name: str, elem_size: int | tuple = 2) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    sizes = elem_size if isinstance(elem_size, tuple) else (elem_size,)
    if t.element_size() not in sizes:
        raise ValueError(f"{name} must have {sizes}-byte elements")


def _per_slot(t: torch.Tensor, batch: int, like: torch.Tensor, name: str = "lr_mul_per_slot") -> None:
    """A per-slot float32 vector: dense, float32, exactly ``batch`` elements, on ``like``'s device (the
    C ABI reads ``batch`` floats from the pointer and cannot check any of this itself)."""
    _dense(t, name, 4)
    if t.dtype != torch.float32:
        raise ValueError(f"{name} must be float32 (got {t.dtype})")
    if t.numel() != batch:
        raise ValueError(f"{name} must have {batch} elements, one per slot (got {t.numel()})")
    if t.device != like.device:
        raise ValueError(f"{name} must be on {like.device} (got {t.device})")


def default_hparams() -> mb_hparams:
    hp = mb_hparams()
    lib().mb_default_hparams(ctypes.byref(hp))
    return hp


def _schedule_array(schedule):
    """[(a, b, c), ...] -> a ctypes array of 3*len doubles."""
    flat = [float(v) for abc in schedule for v in abc]
    if len(flat) != 3 * len(schedule) or not schedule:
        raise ValueError("schedule must be a non-empty sequence of (a, b, c)")
    return (ctypes.c_double * len(flat))(*flat)


def make_hparams(schedule=None, **kw) -> mb_hparams:
    """mb_hparams with the library defaults, overridden by keyword; ``schedule`` = [(a, b, c), ...]
    sets per-round coefficients (and ns_steps to its length).  The returned struct keeps the
    schedule array alive."""
    hp = default_hparams()
    for k, v in kw.items():
        if not hasattr(hp, k) or k in ("ns_schedule", "slot_scalars"):
            raise KeyError(k)
        setattr(hp, k, v)
    if schedule is not None:
        arr = _schedule_array(schedule)
        hp.ns_steps = len(schedule)
        hp.ns_schedule = ctypes.cast(arr, ctypes.c_void_p)
        hp._schedule_keepalive = arr
    return hp


@dataclass
class Bank:
    """One viewed bank [batch, rows, cols] of device tensors."""
    grad: torch.Tensor            # bf16 or fp32
    momentum: torch.Tensor        # same dtype as grad
    w_hi: torch.Tensor            # bf16 weight (2-byte)
    w_lo: torch.Tensor            # uint16 low mantissa (2-byte)
    lr_mul: float = 1.0
    wd_mul: float = 1.0
    lr_mul_per_slot: torch.Tensor | None = None   # float32 [batch]
    v_out: torch.Tensor | None = None             # optional bf16 [batch, rows, cols]
    u_out: torch.Tensor | None = None             # optional bf16 [batch, rows, cols]

    def to_c(self) -> mb_bank:
        g = self.grad
        _dense(g, "grad", (2, 4))
        if g.dim() != 3:
            raise ValueError("grad must be [batch, rows, cols]")
        if g.dtype == torch.float32:
            dt = MB_F32
        elif g.dtype == torch.bfloat16:
            dt = MB_BF16
        else:
            raise ValueError("grad must be float32 or bfloat16")
        if self.momentum.dtype != g.dtype:
            raise ValueError("momentum must have the gradient's dtype")
        for name in ("momentum", "w_hi", "w_lo", "v_out", "u_out"):
            t = getattr(self, name)
            if t is None:
                continue
            _dense(t, name, g.element_size() if name == "momentum" else 2)
            if tuple(t.shape) != tuple(g.shape):
                raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(g.shape)}")
        if self.lr_mul_per_slot is not None:
            _per_slot(self.lr_mul_per_slot, g.shape[0], g)
        b, r, c = g.shape
        return mb_bank(b, r, c, dt, float(self.lr_mul), float(self.wd_mul), _ptr(g), _ptr(self.momentum),
                       _ptr(self.w_hi), _ptr(self.w_lo), _ptr(self.lr_mul_per_slot), _ptr(self.v_out),
                       _ptr(self.u_out))


def slot_scalars_table(banks, hp: mb_hparams | None = None):
    """numpy float32 [total slots, 4]: (mu, nu, decay, eta) of every slot of the banks in order, as the
    step derives them (mb_slot_scalars_fill); edit rows, upload, and pass it with ``with_slot_scalars``."""
    import numpy as np
    cb = [b.to_c() for b in banks]
    arr = (mb_bank * len(cb))(*cb)
    n = sum(int(c.batch) for c in cb)
    out = np.zeros((n, 4), dtype=np.float32)
    _check(lib().mb_slot_scalars_fill(arr, len(cb), ctypes.byref(hp) if hp is not None else None,
                                      out.ctypes.data, out.size))
    return out


def with_slot_scalars(hp: mb_hparams | None, table: torch.Tensor | None) -> mb_hparams:
    """A copy of hp (defaults if None) whose per-slot scalar table is the device tensor ``table``
    (float32 [total slots, 4], contiguous); None clears it.  The struct keeps the tensor alive."""
    out = mb_hparams()
    ctypes.pointer(out)[0] = hp if hp is not None else default_hparams()
    if hp is not None and hasattr(hp, "_schedule_keepalive"):
        out._schedule_keepalive = hp._schedule_keepalive
    if table is None:
        out.slot_scalars = None
        return out
    _dense(table, "slot_scalars", 4)
    if table.dtype != torch.float32 or table.dim() != 2 or table.shape[1] != 4:
        raise ValueError("slot_scalars must be float32 [total slots, 4]")
    out.slot_scalars = table.data_ptr()
    out._slot_scalars_keepalive = table
    return out


def mb_step_workspace_bytes(banks) -> int:
    arr = (mb_bank * len(banks))(*[b.to_c() for b in banks])
    return int(lib().mb_step_workspace_bytes(arr, len(banks)))


def mb_ns_workspace_bytes(batch: int, rows: int, cols: int) -> int:
    return int(lib().mb_ns_workspace_bytes(batch, rows, cols))


def _workspace(nbytes: int, like: torch.Tensor, workspace: torch.Tensor | None) -> torch.Tensor:
    if workspace is None:
        return torch.empty(max(nbytes, 16), dtype=torch.uint8, device=like.device)
    _dense(workspace, "workspace", (1, 2, 4, 8))
    return workspace


def muon_bank_step(banks, hp: mb_hparams | None = None, workspace: torch.Tensor | None = None, stream=None):
    """The full Muon step on a list of ``Bank``s (in place on momentum, w_hi, w_lo)."""
    if isinstance(banks, Bank):
        banks = [banks]
    cbanks = [b.to_c() for b in banks]
    table = getattr(hp, "_slot_scalars_keepalive", None) if hp is not None and hp.slot_scalars else None
    if table is not None and table.shape[0] != sum(int(c.batch) for c in cbanks):
        raise ValueError("slot_scalars must have one row per slot of the banks")
    arr = (mb_bank * len(cbanks))(*cbanks)
    need = int(lib().mb_step_workspace_bytes(arr, len(cbanks)))
    ws = _workspace(need, banks[0].grad, workspace)
    hp_ref = ctypes.byref(hp) if hp is not None else None
    _check(lib().muon_bank_step(arr, len(cbanks), hp_ref, ws.data_ptr(), ws.numel() * ws.element_size(),
                                _stream(stream)))
    return ws


def muon_momentum_update(grad: torch.Tensor, momentum: torch.Tensor, u_out: torch.Tensor, mu: float, nu: float,
                         stream=None) -> None:
    """buf' = RN(mu*buf + nu*g) in place and u = RN_bf16(nu*g + mu*buf') into u_out."""
    _dense(grad, "grad", (2, 4))
    _dense(momentum, "momentum", grad.element_size())
    _dense(u_out, "u_out", 2)
    if grad.dtype not in (torch.float32, torch.bfloat16) or momentum.dtype != grad.dtype:
        raise ValueError("grad/momentum must both be float32 or both bfloat16")
    if grad.dim() != 3 or momentum.shape != grad.shape or u_out.shape != grad.shape:
        raise ValueError("grad, momentum and u_out must be [batch, rows, cols] of one shape")
    b, r, c = grad.shape
    dt = MB_F32 if grad.dtype == torch.float32 else MB_BF16
    _check(lib().muon_momentum_update(_ptr(grad), _ptr(momentum), _ptr(u_out), b, r, c, dt, float(mu), float(nu),
                                      _stream(stream)))


def ns_orthogonalize_batched(x: torch.Tensor, y: torch.Tensor | None = None, steps: int = 5, a: float = 3.4445,
                             b: float = -4.7750, c: float = 2.0315, eps: float = 1e-7,
                             workspace: torch.Tensor | None = None, stream=None, schedule=None) -> torch.Tensor:
    """y = NS(x) for bf16 [batch, rows, cols]; returns y (a new tensor if none is given).
    ``schedule`` = [(a, b, c), ...] gives every round its own coefficients (steps = its length)."""
    _dense(x, "x", 2)
    if x.dim() != 3:
        raise ValueError("x must be [batch, rows, cols]")
    if y is None:
        y = torch.empty_like(x)
    _dense(y, "y", 2)
    if y.shape != x.shape:
        raise ValueError("y must have x's shape")
    bt, r, cc = x.shape
    ws = _workspace(int(lib().mb_ns_workspace_bytes(bt, r, cc)), x, workspace)
    if schedule is not None:
        arr = _schedule_array(schedule)
        _check(lib().ns_orthogonalize_batched_sched(_ptr(x), _ptr(y), bt, r, cc, len(schedule), ctypes.cast(arr, vp_t),
                                                    float(eps), ws.data_ptr(), ws.numel() * ws.element_size(),
                                                    _stream(stream)))
        return y
    _check(lib().ns_orthogonalize_batched(_ptr(x), _ptr(y), bt, r, cc, int(steps), float(a), float(b), float(c),
                                          float(eps), ws.data_ptr(), ws.numel() * ws.element_size(), _stream(stream)))
    return y


def ns_orthogonalize_batched_noalloc(x: torch.Tensor, y: torch.Tensor, steps: int = 5, a: float = 3.4445,
                                     b: float = -4.7750, c: float = 2.0315, eps: float = 1e-7, stream=None) -> None:
    """y = NS(x) for bf16 [batch, rows, cols] with the library's static scratch: nothing is allocated here
    or in the library (y must be given; it may be x)."""
    _dense(x, "x", 2)
    _dense(y, "y", 2)
    if x.dim() != 3 or y.shape != x.shape:
        raise ValueError("x and y must be [batch, rows, cols] of one shape")
    bt, r, cc = x.shape
    _check(lib().ns_orthogonalize_batched_noalloc(_ptr(x), _ptr(y), bt, r, cc, int(steps), float(a), float(b),
                                                  float(c), float(eps), _stream(stream)))


def mp_apply_update(w_hi: torch.Tensor, w_lo: torch.Tensor, v: torch.Tensor, eff_lr: float, decay: float,
                    lr_mul_per_slot: torch.Tensor | None = None, stream=None) -> None:
    """In place on (w_hi, w_lo): w = fp32(hi, lo); r = RN32(RN32(w*decay) - eta*v); split r.
    The leading dimension is the slot (for the optional per-slot multiplier)."""
    for t, n in ((w_hi, "w_hi"), (w_lo, "w_lo"), (v, "v")):
        _dense(t, n, 2)
    if w_lo.shape != w_hi.shape or v.shape != w_hi.shape:
        raise ValueError("w_hi, w_lo and v must have one shape")
    batch = w_hi.shape[0] if w_hi.dim() > 1 else 1
    slot = w_hi.numel() // max(batch, 1)
    if lr_mul_per_slot is not None:
        _per_slot(lr_mul_per_slot, batch, w_hi)
    _check(lib().mp_apply_update(_ptr(w_hi), _ptr(w_lo), _ptr(v), batch, slot, float(eff_lr), float(decay),
                                 _ptr(lr_mul_per_slot), _stream(stream)))


def transpose_copy(dst: torch.Tensor, src: torch.Tensor, stream=None) -> None:
    """dst [cols, rows] = src [rows, cols] transposed (bits copied; 2- or 4-byte elements)."""
    if src.dim() != 2 or dst.shape != (src.shape[1], src.shape[0]) or dst.element_size() != src.element_size():
        raise ValueError("dst must be src's transpose shape with the same element size")
    _dense(src, "src", (2, 4))
    _dense(dst, "dst", src.element_size())
    _check(lib().transpose_copy(_ptr(dst), _ptr(src), src.shape[0], src.shape[1], src.element_size(), _stream(stream)))


def transpose_add(dst: torch.Tensor, src: torch.Tensor, stream=None) -> None:
    """dst [cols, rows] += src [rows, cols] transposed, one rounding (float32 or bfloat16)."""
    if src.dim() != 2 or dst.shape != (src.shape[1], src.shape[0]) or dst.dtype != src.dtype:
        raise ValueError("dst must be src's transpose shape with the same dtype")
    if src.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("transpose_add takes float32 or bfloat16")
    _dense(src, "src", (2, 4))
    _dense(dst, "dst", src.element_size())
    dt = MB_F32 if src.dtype == torch.float32 else MB_BF16
    _check(lib().transpose_add(_ptr(dst), _ptr(src), src.shape[0], src.shape[1], dt, _stream(stream)))


def mb_ns_set_path(path: int) -> int:
    """0: persistent Newton-Schulz launch where the shape allows it; 1: one launch per contraction.
    Returns the previous setting."""
    prev = lib().mb_ns_set_path(int(path))
    if prev < 0:
        raise ValueError(f"unknown Newton-Schulz path {path}")
    return prev


def mb_device_fault(clear: bool = False) -> bool:
    """Whether a persistent Newton-Schulz launch on the current device gave up a dependency wait at its
    time cap since the flag was last cleared (blocking; synchronize the step's streams first)."""
    r = lib().mb_device_fault(1 if clear else 0)
    if r < 0:
        raise MuonBankError(8, lib().mb_last_error().decode())
    return r == 1


def mb_test_persist_faults(wait_cap_ticks: int = 0, extra_queues: int = 0) -> None:
    """Test hook for the persistent launch's failure paths (tests only): a dependency-wait cap in ticks of
    the 100 MHz constant clock (0: the default 200 ms) and extra XCD queues that no workgroup serves."""
    _check(lib().mb_test_persist_faults(int(wait_cap_ticks), int(extra_queues)))


def mb_timing_enable(on: bool) -> None:
    lib().mb_timing_enable(1 if on else 0)


def mb_timing_read() -> dict:
    """{kernel name: (launches, total ms)} for the launches timed since the last read."""
    buf = (mb_kernel_time * 64)()
    n = lib().mb_timing_read(buf, 64)
    if n < 0:
        raise MuonBankError(8, "timing read failed")
    return {buf[i].name.decode(): (int(buf[i].launches), float(buf[i].total_ms)) for i in range(min(n, 64))}
