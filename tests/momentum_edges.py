"""Constructed inputs for the momentum + Nesterov rounding, one regime per case family.

With mu = 0.75 and nu = 0.25 (exact in float32) the products mu*b of short significands land exactly on
rounding midpoints of the storage format, so the cases reach every branch of a correctly rounded sum
evaluated through binary64:

  tie      the exact sum is a midpoint (round half to even);
  sticky   the exact sum is a midpoint plus a term far below binary64's resolution: its binary64 sum is
           the midpoint itself, and only the sign of the lost term decides (2^-58 relative);
  select   the exact sum is a midpoint plus a term binary64 keeps but float32 loses (2^-40 relative);
  cancel   mu*b and nu*g cancel to a few bits;
  tiny     results in the subnormal range of the storage format;
  random   ordinary values, both signs, several binades.

The "u" families do the same for the second sum u = nu*g + mu*buf', through a buffer value buf' whose
product with mu is a bf16 midpoint.  Every value is exactly representable in the storage format (bf16
bits or float32).  No arithmetic of the method is here: expected results come from the oracle.
"""

from __future__ import annotations

import numpy as np

MU, NU = 0.75, 0.25


def _bf16(x) -> np.ndarray:
    """float64 values that are exact bf16 -> bf16 bits (raises if one is not)."""
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    if not np.array_equal(f.astype(np.float64), np.asarray(x, dtype=np.float64)):
        raise ValueError("not exact in float32")
    b = f.view(np.uint32)
    if np.any(b & np.uint32(0xFFFF)):
        raise ValueError("not exact in bf16")
    return (b >> np.uint32(16)).astype(np.uint16)


def _f32(x) -> np.ndarray:
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    if not np.array_equal(f.astype(np.float64), np.asarray(x, dtype=np.float64)):
        raise ValueError("not exact in float32")
    return f


# b = (1 + k/128) 2^e makes mu*b = 0.75 b a bf16 midpoint: for odd k up to 41 it lies in [0.75, 1), where
# midpoints are odd multiples of 2^-9; for k = 2 mod 4 from 44 on in [1, 1.5), odd multiples of 2^-8
_MID_K = np.array([k for k in range(1, 128) if (k % 2 == 1 and k <= 41) or (k % 4 == 2 and k >= 44)])


def bf16_cases(seed: int = 11):
    """(families, g, b) for bf16 storage: families maps a family name to its index range; g and b are
    float64 values exact in bf16."""
    rng = np.random.default_rng(seed)
    g, b, fam = [], [], {}

    def add(name, gs, bs):
        start = len(g)
        g.extend(gs)
        b.extend(bs)
        fam[name] = (start, len(g))

    odd = _MID_K
    for e in (-60, -20, 0, 20, 100):
        for sgn in (1.0, -1.0):
            mid_b = sgn * (1.0 + odd / 128.0) * 2.0 ** e           # mu*b is a bf16 midpoint
            add(f"tie e{e} s{sgn:+.0f}", [0.0] * odd.size, mid_b)
            for d in (1.0, -1.0):
                add(f"sticky e{e} s{sgn:+.0f} d{d:+.0f}", [d * 2.0 ** (e - 56)] * odd.size, mid_b)
                add(f"select e{e} s{sgn:+.0f} d{d:+.0f}", [d * 2.0 ** (e - 40)] * odd.size, mid_b)
    # the second sum: buf' = B with mu*B a bf16 midpoint, reached from b = B/mu (b exact in bf16 when
    # B/mu is; else the nearest bf16 whose first sum still rounds to B)
    for e in (-20, 0, 20):
        for sgn in (1.0, -1.0):
            B = sgn * (1.0 + odd / 128.0) * 2.0 ** e
            bb = np.array([float(np.float32(v)) for v in B / MU])
            bb = np.array([float(_bf16_round(v)) for v in bb])
            add(f"u tie e{e} s{sgn:+.0f}", [0.0] * odd.size, bb)
            for d in (1.0, -1.0):
                add(f"u sticky e{e} s{sgn:+.0f} d{d:+.0f}", [d * 2.0 ** (e - 56)] * odd.size, bb)
                add(f"u select e{e} s{sgn:+.0f} d{d:+.0f}", [d * 2.0 ** (e - 40)] * odd.size, bb)
    # cancellation: nu*g = -mu*b + a few bits
    mags = (1.0 + rng.integers(0, 128, 256) / 128.0) * 2.0 ** rng.integers(-30, 30, 256)
    sg = rng.choice([-1.0, 1.0], 256)
    bb = sg * mags
    gg = np.array([float(_bf16_round(v)) for v in -3.0 * bb * (1.0 + rng.integers(-3, 4, 256) * 2.0 ** -7)])
    add("cancel", gg, bb)
    # subnormal results (bf16 subnormals are below 2^-126)
    k = rng.integers(1, 128, 256)
    add("tiny", rng.choice([-1.0, 1.0], 256) * rng.integers(1, 128, 256) * 2.0 ** -133,
        rng.choice([-1.0, 1.0], 256) * k * 2.0 ** -133)
    # ordinary values
    add("random", [float(_bf16_round(v)) for v in rng.standard_normal(512) * 2.0 ** rng.integers(-40, 40, 512)],
        [float(_bf16_round(v)) for v in rng.standard_normal(512) * 2.0 ** rng.integers(-40, 40, 512)])
    return fam, np.array(g), np.array(b)


def f32_cases(seed: int = 12):
    """(families, g, b) for float32 storage."""
    rng = np.random.default_rng(seed)
    g, b, fam = [], [], {}

    def add(name, gs, bs):
        start = len(g)
        g.extend(gs)
        b.extend(bs)
        fam[name] = (start, len(g))

    k = 2 * rng.integers(0, (1 << 23) // 6, 64) + 1               # odd, and 0.75 b stays below 1
    for e in (-60, 0, 60):
        for sgn in (1.0, -1.0):
            mid_b = sgn * (1.0 + k * 2.0 ** -23) * 2.0 ** e            # mu*b is a float32 midpoint
            add(f"tie e{e} s{sgn:+.0f}", [0.0] * k.size, mid_b)
            for d in (1.0, -1.0):
                add(f"sticky e{e} s{sgn:+.0f} d{d:+.0f}", [d * 2.0 ** (e - 60)] * k.size, mid_b)
    odd = _MID_K
    for e in (-20, 0, 20):
        for sgn in (1.0, -1.0):
            B = sgn * (1.0 + odd / 128.0) * 2.0 ** e                   # mu*B is a bf16 midpoint
            bb = np.array([float(np.float32(v)) for v in B / MU])
            add(f"u tie e{e} s{sgn:+.0f}", [0.0] * odd.size, bb)
            for d in (1.0, -1.0):
                add(f"u sticky e{e} s{sgn:+.0f} d{d:+.0f}", [d * 2.0 ** (e - 56)] * odd.size, bb)
                add(f"u select e{e} s{sgn:+.0f} d{d:+.0f}", [d * 2.0 ** (e - 40)] * odd.size, bb)
    add("tiny", rng.choice([-1.0, 1.0], 256) * rng.integers(1, 1 << 20, 256) * 2.0 ** -149,
        rng.choice([-1.0, 1.0], 256) * rng.integers(1, 1 << 20, 256) * 2.0 ** -149)
    add("random", [float(np.float32(v)) for v in rng.standard_normal(512) * 2.0 ** rng.integers(-40, 40, 512)],
        [float(np.float32(v)) for v in rng.standard_normal(512) * 2.0 ** rng.integers(-40, 40, 512)])
    return fam, np.array(g), np.array(b)


def _bf16_round(v: float) -> np.float32:
    """A bf16 value near v (round half away on the 16 dropped bits; only used to make inputs)."""
    f = np.float32(v)
    u = np.array([f]).view(np.uint32)[0]
    u = (int(u) + 0x8000) & 0xFFFF0000
    return np.array([u], dtype=np.uint32).view(np.float32)[0]


def as_bank(values: np.ndarray, cols: int, fmt: str):
    """Pad to a whole number of rows of `cols` and shape as one slot [1, rows, cols] (bf16 bits or float32)."""
    n = values.size
    rows = -(-n // cols)
    pad = np.zeros(rows * cols, dtype=np.float64)
    pad[:n] = values
    arr = _bf16(pad) if fmt == "bf16" else _f32(pad)
    return arr.reshape(1, rows, cols)
