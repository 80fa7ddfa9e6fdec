"""Binding of the measurement probes in libmuonbank.so (``include/muonbank_probes.h``): argument
marshalling only.  The benchmark times them to report fractions of the measured peaks beside the
nominal ones."""

from __future__ import annotations

import ctypes

import torch

from . import api

EXPORTED = ("mb_probe_mfma_bf16", "mb_probe_copy")
MFMA_FLOPS = 2 * 32 * 32 * 16          # one v_mfma_f32_32x32x16_bf16
WAVES_PER_WORKGROUP = 4
CHAINS = 4

_bound = False


def _lib():
    global _bound
    L = api.lib()
    if not _bound:
        vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
        L.mb_probe_mfma_bf16.restype = i32
        L.mb_probe_mfma_bf16.argtypes = [i64, i32, vp, vp]
        L.mb_probe_copy.restype = i32
        L.mb_probe_copy.argtypes = [vp, vp, i64, vp]
        _bound = True
    return L


def mfma_flops(iters: int, workgroups: int) -> int:
    return workgroups * WAVES_PER_WORKGROUP * iters * CHAINS * MFMA_FLOPS


def mb_probe_mfma_bf16(iters: int, workgroups: int, sink: torch.Tensor, stream=None) -> None:
    api._dense(sink, "sink", 4)
    if sink.numel() < workgroups * 256:
        raise ValueError("sink must hold workgroups * 256 floats")
    api._check(_lib().mb_probe_mfma_bf16(int(iters), int(workgroups), sink.data_ptr(), api._stream(stream)))


def mb_probe_copy(dst: torch.Tensor, src: torch.Tensor, stream=None) -> None:
    api._dense(dst, "dst", (1, 2, 4, 8))
    api._dense(src, "src", (1, 2, 4, 8))
    n = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() < n:
        raise ValueError("dst is smaller than src")
    api._check(_lib().mb_probe_copy(dst.data_ptr(), src.data_ptr(), n, api._stream(stream)))
