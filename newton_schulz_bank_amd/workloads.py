"""Seeded synthetic inputs for the Muon bank step.

This module only draws and quantises random inputs; it holds none of the
step's arithmetic.  The tests, the benchmark and the smoke check draw their
inputs here, and the same host arrays are handed to the HIP library and to
the CPU oracle.

The shapes are the stacked parameter banks of the modded-nanogpt records,
viewed zero-copy as [batch, rows, cols] ("Unified zero-copy optimizer and
transposed LM head", section 1.1):

* attention QKVO bank (10, 4*768, 768) -> (40, 768, 768);
* MLP bank (12, 2, 3072, 768) -> (24, 3072, 768), whose last slot is padding;
* the later MLP bank (12, 2, 2816, 768) -> (24, 2816, 768), with MLP layer 7
  dead, i.e. view slots 14 and 15 (the page counts that slot on the 12-layer
  index); workload 7 takes the other reading, view slot 7 dead, on the same
  random draws;
* the 350M-scale banks (24, 4096, 1024) -> (96, 1024, 1024) and
  (24, 2, 4096, 1024) -> (48, 4096, 1024);
* the gate matrices smear_gate (1 live of 16) and attn_gate (10 live of 16)
  ("Muon Custom Sizing", section 2.1 counts their padding);
* one rank's share of the big banks when the slot axis is split over 8 GPUs
  (5 attention and 3 MLP slots per GPU at 124M, "Unified zero-copy optimizer
  and transposed LM head", section 1.1; 12 + 6 + 3 slots at 350M): the
  kernels at the shape one GPU of that schedule runs.

Distributions: N(0, s) means standard deviation s, drawn in float64, rounded
to float32 and then (for bf16 tensors) to bf16, both round-to-nearest-even.
Low mantissas are uniform on [0, 65535].  Heavy-tailed gradients are
1e-3 * Student-t with 3 degrees of freedom.  Dead slots are all-zero in every
tensor.  Seed of a tensor = 1000*(config+1) + 10*bank + tensor id (grad 1,
momentum 2, weight 3, mantissa 4), PCG64.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

GRAD, MOMENTUM, WEIGHT, MANTISSA = 1, 2, 3, 4


@dataclass(frozen=True)
class BankSpec:
    name: str
    batch: int
    rows: int
    cols: int
    grad_dtype: str = "bf16"          # "bf16" or "f32"; the momentum buffer has the same dtype
    grad_dist: str = "normal"         # "normal" or "student_t3"
    grad_scale: float = 1e-3
    mom_scale: float | None = 1e-3    # None = zero buffer
    w_scale: float = 0.02
    lo_uniform: bool = True           # False = zero mantissa
    dead_slots: tuple = field(default_factory=tuple)
    seed_config: int | None = None    # draw with another workload's seeds (None = this workload's)

    @property
    def numel(self) -> int:
        return self.batch * self.rows * self.cols

    @property
    def live_slots(self) -> tuple:
        return tuple(i for i in range(self.batch) if i not in self.dead_slots)


def _attn(batch=40, d=768):
    return BankSpec("attn_qkvo", batch, d, d)


WORKLOADS: dict[int, list[BankSpec]] = {
    0: [BankSpec("fp32_256", 4, 256, 256, grad_dtype="f32", grad_scale=1.0, mom_scale=None,
                 lo_uniform=False)],
    1: [_attn()],
    2: [BankSpec("mlp_3072", 24, 3072, 768, dead_slots=(23,))],
    3: [_attn(),
        BankSpec("mlp_3072", 24, 3072, 768, dead_slots=(23,)),
        BankSpec("smear_gate", 16, 1, 12, dead_slots=tuple(range(1, 16))),
        BankSpec("attn_gate", 16, 6, 12, dead_slots=tuple(range(10, 16)))],
    4: [BankSpec("attn_1024", 96, 1024, 1024, grad_dist="student_t3"),
        BankSpec("mlp_4096", 48, 4096, 1024, grad_dist="student_t3"),
        BankSpec("mlp_2816", 24, 2816, 768, grad_dist="student_t3", dead_slots=(14, 15))],
    # one rank's slots of the 124M and of the 350M banks on 8 GPUs (rank 0: every slot live)
    5: [_attn(batch=5), BankSpec("mlp_3072", 3, 3072, 768)],
    6: [BankSpec("attn_1024", 12, 1024, 1024, grad_dist="student_t3"),
        BankSpec("mlp_4096", 6, 4096, 1024, grad_dist="student_t3"),
        BankSpec("mlp_2816", 3, 2816, 768, grad_dist="student_t3")],
    # workload 4 with the other reading of the 2816 bank's dead MLP: view slot 7 (same draws as 4)
    7: [BankSpec("attn_1024", 96, 1024, 1024, grad_dist="student_t3", seed_config=4),
        BankSpec("mlp_4096", 48, 4096, 1024, grad_dist="student_t3", seed_config=4),
        BankSpec("mlp_2816", 24, 2816, 768, grad_dist="student_t3", dead_slots=(7,), seed_config=4)],
}

WORKLOAD_NAMES = {
    0: "4x256x256 fp32 grads, zero momentum",
    1: "attention QKVO bank (10,3072,768) viewed (40,768,768)",
    2: "MLP bank (12,2,3072,768) viewed (24,3072,768), slot 23 dead",
    3: "124M optimizer step: attn (40,768,768) + MLP (24,3072,768) + gates (16,1,12), (16,6,12)",
    4: "350M banks (96,1024,1024) + (48,4096,1024) + (24,2816,768) slots 14-15 dead",
    5: "one GPU's share of the 124M banks on 8 GPUs: attn (5,768,768) + MLP (3,3072,768)",
    6: "one GPU's share of the 350M banks on 8 GPUs: (12,1024,1024) + (6,4096,1024) + (3,2816,768)",
    7: "350M banks (96,1024,1024) + (48,4096,1024) + (24,2816,768) view slot 7 dead",
}


def _rng(config: int, bank: int, tensor: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(1000 * (config + 1) + 10 * bank + tensor))


def _to_bf16_bits(x64: np.ndarray) -> np.ndarray:
    """float64 samples -> float32 (RN-even) -> bf16 bits (RN-even), via torch's CPU cast."""
    import torch
    f32 = torch.from_numpy(np.ascontiguousarray(x64, dtype=np.float32))
    return f32.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def _sample(rng, dist, scale, shape):
    if dist == "normal":
        return rng.normal(0.0, scale, size=shape)
    if dist == "student_t3":
        return scale * rng.standard_t(3, size=shape)
    raise ValueError(dist)


def _zero_dead(arr: np.ndarray, dead: tuple) -> np.ndarray:
    if dead:
        arr[list(dead)] = 0
    return arr


def make_bank(config: int, bank: int, spec: BankSpec | None = None, slots=None) -> dict:
    """Draw one bank's inputs.

    Returns a dict with ``grad`` and ``momentum`` (uint16 bf16 bits, or float32
    for fp32 banks), ``w_hi`` (uint16 bf16 weight bits) and ``w_lo`` (uint16
    low mantissas), each of shape [batch, rows, cols].  ``slots`` (optional)
    keeps only the listed slots of the full draw, for small samples of big banks."""
    spec = spec or WORKLOADS[config][bank]
    shape = (spec.batch, spec.rows, spec.cols)
    sc = config if spec.seed_config is None else spec.seed_config
    g64 = _sample(_rng(sc, bank, GRAD), spec.grad_dist, spec.grad_scale, shape)
    if spec.mom_scale is None:
        m64 = np.zeros(shape)
    else:
        m64 = _rng(sc, bank, MOMENTUM).normal(0.0, spec.mom_scale, size=shape)
    w64 = _rng(sc, bank, WEIGHT).normal(0.0, spec.w_scale, size=shape)
    if spec.lo_uniform:
        lo = _rng(sc, bank, MANTISSA).integers(0, 65536, size=shape, dtype=np.uint32).astype(np.uint16)
    else:
        lo = np.zeros(shape, dtype=np.uint16)
    if spec.grad_dtype == "f32":
        grad = g64.astype(np.float32)
        mom = m64.astype(np.float32)
    else:
        grad = _to_bf16_bits(g64)
        mom = _to_bf16_bits(m64)
    del g64, m64
    w_hi = _to_bf16_bits(w64)
    del w64
    out = {"grad": grad, "momentum": mom, "w_hi": w_hi, "w_lo": lo}
    for k in out:
        _zero_dead(out[k], spec.dead_slots)
    if slots is not None:
        out = {k: np.ascontiguousarray(v[list(slots)]) for k, v in out.items()}
    return out


def make_random_bank(seed: int, batch: int, rows: int, cols: int, grad_dtype: str = "bf16",
                     grad_scale: float = 1e-3, mom_scale: float | None = 1e-3, w_scale: float = 0.02,
                     dead_slots=()) -> dict:
    """Same recipe as ``make_bank`` for an arbitrary shape (parity cases with
    ragged or tiny shapes), seeded directly."""
    spec = BankSpec("custom", batch, rows, cols, grad_dtype=grad_dtype, grad_scale=grad_scale,
                    mom_scale=mom_scale, w_scale=w_scale, dead_slots=tuple(dead_slots))
    shape = (batch, rows, cols)
    rng = np.random.Generator(np.random.PCG64(seed))
    g64 = rng.normal(0.0, grad_scale, size=shape)
    m64 = np.zeros(shape) if mom_scale is None else rng.normal(0.0, mom_scale, size=shape)
    w64 = rng.normal(0.0, w_scale, size=shape)
    lo = rng.integers(0, 65536, size=shape, dtype=np.uint32).astype(np.uint16)
    if grad_dtype == "f32":
        grad, mom = g64.astype(np.float32), m64.astype(np.float32)
    else:
        grad, mom = _to_bf16_bits(g64), _to_bf16_bits(m64)
    out = {"grad": grad, "momentum": mom, "w_hi": _to_bf16_bits(w64), "w_lo": lo}
    for k in out:
        _zero_dead(out[k], spec.dead_slots)
    return out


def random_bf16_matrices(seed: int, batch: int, rows: int, cols: int, scale: float = 1.0) -> np.ndarray:
    """bf16 bits of N(0, scale) matrices, for the stand-alone Newton-Schulz entry point."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return _to_bf16_bits(rng.normal(0.0, scale, size=(batch, rows, cols)))


def conditioned_bf16_matrices(seed: int, batch: int, rows: int, cols: int,
                              smin: float = 0.5, smax: float = 1.0) -> np.ndarray:
    """bf16 bits of Q1 diag(s) Q2^T with random orthogonal Q1, Q2 and singular
    values s uniform on [smin, smax]: well-conditioned inputs whose Newton-Schulz
    output must land in the iteration's fixed band."""
    rng = np.random.Generator(np.random.PCG64(seed))
    m = min(rows, cols)
    out = np.empty((batch, rows, cols))
    for i in range(batch):
        q1, _ = np.linalg.qr(rng.normal(size=(rows, m)))
        q2, _ = np.linalg.qr(rng.normal(size=(cols, m)))
        s = rng.uniform(smin, smax, size=m)
        out[i] = (q1 * s) @ q2.T
    return _to_bf16_bits(out)
