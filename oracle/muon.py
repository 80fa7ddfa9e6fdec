"""Plain float64 oracle of the Muon bank step (test infrastructure only).

The step, per viewed bank [batch, rows, cols] (zero-copy views of the stacked
banks, "Unified zero-copy optimizer and transposed LM head", section 1.1):

1. momentum lerp   buf' = mu*buf + (1-mu)*g        ("Muon Custom Sizing", section 4)
2. Nesterov lerp   u    = (1-mu)*g + mu*buf'       (same section; "nesterov" in the
                                                     "four optimizers" section of the
                                                     U-Net page)
3. Newton-Schulz   v    = NS5(u) in bf16            ("Muon Custom Sizing", section 2.3;
                                                     Record 7 page, section 4.2)
4. mixed-precision apply on the fp32 master made of the bf16 weight (high half)
   and a uint16 low mantissa: w <- w*(1 - lr*wd*wd_mul) - eta*v, split back
   (Record 7 page, section 4.1), with eta = lr*sqrt(max(1, rows/cols))*lr_mul
   ("Muon Custom Sizing", section 4; U-Net page, "four optimizers").

Rounding is stated exactly so that integer and storage bits can be compared
bit for bit:

* host scalars are evaluated in float64 and rounded once to float32;
* buf' and u are the exact values rounded once (round-to-nearest-even) to the
  storage format (bf16, or fp32 for fp32 gradients);
* the apply rounds exactly twice: t = RN32(w*d), then r = RN32(t - eta*v)
  with the product eta*v unrounded;
* the mantissa split is a bit slice (truncation), not a rounding.

Exact rounding uses float64 where the float64 result is provably exact
(products of two <=24-bit significands) and ``fractions.Fraction`` for the
rare sums that float64 cannot hold exactly (detected with Knuth's TwoSum).
"""

from __future__ import annotations

import math
from dataclasses import dataclass
from fractions import Fraction

import numpy as np

BF16 = "bf16"
F32 = "f32"

# (significand bits incl. the implicit one, minimum normal exponent, maximum exponent)
_FORMATS = {
    BF16: (8, -126, 127),
    F32: (24, -126, 127),
}


# ---------------------------------------------------------------------------
# rounding to a binary format
# ---------------------------------------------------------------------------

def _pow2(k: int) -> Fraction:
    return Fraction(2) ** k


def round_fraction(q: Fraction, p: int, emin: int, emax: int) -> float:
    """Round the exact rational ``q`` to the nearest value of the binary format
    with a ``p``-bit significand (normal exponents emin..emax, gradual underflow),
    ties to even; results beyond the largest finite value become +-inf."""
    if q == 0:
        return 0.0
    neg = q < 0
    a = -q if neg else q
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if _pow2(e) > a:
        e -= 1
    # now 2**e <= a < 2**(e+1)
    quantum = _pow2(max(e, emin) - (p - 1))
    n = a / quantum
    whole = n.numerator // n.denominator
    rest = n - whole
    if rest > Fraction(1, 2) or (rest == Fraction(1, 2) and whole % 2 == 1):
        whole += 1
    val = whole * quantum
    max_finite = (2 - _pow2(1 - p)) * _pow2(emax)
    if val > max_finite:
        return -math.inf if neg else math.inf
    out = float(val)
    return -out if neg else out


def round_to_format(x, p: int, emin: int, emax: int) -> np.ndarray:
    """Round every float64 in ``x`` to the nearest value of the binary format
    (p-bit significand, gradual underflow below 2**emin), ties to even.

    The value is put on the grid of its binade -- spacing 2**(e-p+1) with
    e = max(floor(log2|x|), emin) -- and rounded to the nearest grid point by
    ``np.rint`` (ties to even).  Division by a power of two is exact."""
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)
    ex = np.maximum(e.astype(np.int64) - 1, emin)
    quantum = np.ldexp(1.0, (ex - (p - 1)).astype(np.int32))
    with np.errstate(over="ignore", invalid="ignore"):
        y = np.rint(x / quantum) * quantum
    max_finite = math.ldexp(2.0 - 2.0 ** (1 - p), emax)
    y = np.where(np.abs(y) > max_finite, np.copysign(np.inf, x), y)
    return np.where(np.isfinite(x), y, x)


def round_to_bf16(x) -> np.ndarray:
    """RN-even to bfloat16 (8-bit significand, fp32 exponent range)."""
    return round_to_format(x, *_FORMATS[BF16])


def round_to_f32(x) -> np.ndarray:
    """RN-even to IEEE binary32."""
    return round_to_format(x, *_FORMATS[F32])


def bf16_bits_to_f64(bits) -> np.ndarray:
    """bf16 bit patterns (uint16) -> their values as float64."""
    b = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def f64_to_bf16_bits(x) -> np.ndarray:
    """float64 values that bf16 represents exactly -> their uint16 bit patterns."""
    f = np.ascontiguousarray(x, dtype=np.float64).astype(np.float32)
    bits = f.view(np.uint32)
    if np.any((bits & np.uint32(0xFFFF)) != 0):
        raise ValueError("value is not representable in bf16")
    return (bits >> np.uint32(16)).astype(np.uint16)


def _round_sum_of_products(c1, x1, c2, x2, fmt: str) -> np.ndarray:
    """RN_fmt(c1*x1 + c2*x2), correctly rounded, for float32 coefficients c1, c2
    (scalars, or arrays that broadcast against x1, e.g. one per slot) and arrays
    x1, x2 of fp32 or bf16 values.

    Each product of two <=24-bit significands is exact in float64; the sum is
    exact unless TwoSum reports a nonzero error, and those few elements are
    redone in exact rational arithmetic."""
    p, emin, emax = _FORMATS[fmt]
    x1 = np.asarray(x1, dtype=np.float64)
    x2 = np.asarray(x2, dtype=np.float64)
    c1 = np.broadcast_to(np.asarray(c1, dtype=np.float64), x1.shape)
    c2 = np.broadcast_to(np.asarray(c2, dtype=np.float64), x2.shape)
    p1 = c1 * x1
    p2 = c2 * x2
    s = p1 + p2
    bb = s - p1
    err = (p1 - (s - bb)) + (p2 - bb)
    out = round_to_format(s, p, emin, emax)
    for idx in zip(*np.nonzero((err != 0) & np.isfinite(s))):
        q = Fraction(float(c1[idx])) * Fraction(float(x1[idx])) + Fraction(float(c2[idx])) * Fraction(float(x2[idx]))
        out[idx] = round_fraction(q, p, emin, emax)
    return out


# ---------------------------------------------------------------------------
# host scalars
# ---------------------------------------------------------------------------

@dataclass(frozen=True)
class StepScalars:
    """The per-bank float32 scalars, each evaluated in float64 and rounded once."""
    mu: float      # momentum coefficient
    nu: float      # 1 - mu
    decay: float   # 1 - lr*wd*wd_mul              (decoupled weight decay)
    eta: float     # lr*sqrt(max(1, rows/cols))*lr_mul  (shape-scaled learning rate)


def _f32(v: float) -> float:
    return float(np.float32(v))


def step_scalars(lr: float, weight_decay: float, momentum: float, rows: int, cols: int,
                 lr_mul: float = 1.0, wd_mul: float = 1.0) -> StepScalars:
    """eff_lr = lr * max(1, rows/cols)**0.5 * lr_mul and eff_wd = lr * wd * wd_mul
    ("Muon Custom Sizing", section 4; the U-Net page's "four optimizers" section
    writes the shape factor as max(1, g.size(0)/g.size(1))**0.5).  The decay
    factor is 1 - eff_wd (Record 7 page, section 4.1).  Products are taken left to
    right in float64."""
    return StepScalars(
        mu=_f32(momentum),
        nu=_f32(1.0 - momentum),
        decay=_f32(1.0 - lr * weight_decay * wd_mul),
        eta=_f32(lr * math.sqrt(max(1.0, rows / cols)) * lr_mul),
    )


# ---------------------------------------------------------------------------
# momentum and Nesterov update
# ---------------------------------------------------------------------------

def momentum_nesterov(grad, buf, mu, nu, storage: str):
    """buf' = mu*buf + nu*g  (the buffer's lerp toward g with weight 1-mu), then
    u = nu*g + mu*buf'       (g's lerp toward the *stored* buf' with weight mu)
    ("Muon Custom Sizing", section 4).  buf' is rounded once to the storage
    format, u once to bf16.  mu and nu are float32 values, scalars or arrays
    that broadcast against the bank (one per slot: [batch, 1, 1]).  Returns
    (buf', u) as float64 arrays."""
    buf_new = _round_sum_of_products(mu, buf, nu, grad, storage)
    u = _round_sum_of_products(nu, grad, mu, buf_new, BF16)
    return buf_new, u


# ---------------------------------------------------------------------------
# Newton-Schulz
# ---------------------------------------------------------------------------

NS_COEFFS = (3.4445, -4.7750, 2.0315)
NS_STEPS = 5
NS_EPS = 1e-7


def frobenius_prescale(x, eps: float = NS_EPS) -> np.ndarray:
    """X / (||X||_F + eps): the norm scaling done once before iterating
    ("Muon Custom Sizing", section 2.3 asks for a norm scaling first; the
    Frobenius norm bounds the spectral norm, so every singular value ends
    at most 1)."""
    x = np.asarray(x, dtype=np.float64)
    return x / (math.sqrt(float(np.sum(x * x))) + eps)


def newton_schulz(u, steps: int = NS_STEPS, a: float = NS_COEFFS[0], b: float = NS_COEFFS[1],
                  c: float = NS_COEFFS[2], eps: float = NS_EPS, schedule=None) -> np.ndarray:
    """Quintic Newton-Schulz on every slot of u [batch, rows, cols].

    Per slot: work on X = u (or u^T when rows > cols, so that the Gram matrix
    is the small one), scale by the Frobenius norm, then ``steps`` times
        A = X X^T,   B = b*A + c*A A,   X = a*X + B X,
    the odd quintic a*s + b*s^3 + c*s^5 on the singular values ("Muon Custom
    Sizing", section 2.3: coefficients 3.4445, -4.7750, 2.0315, five rounds;
    Record 7 page, section 4.2: five quintic iterations).  Transposed back at
    the end.  float64 throughout.

    ``schedule``, if given, is a sequence of (a, b, c), one per round: round t
    uses its own coefficients and the number of rounds is len(schedule).  The
    pages name orthogonalizers with per-round coefficients ("Unified zero-copy
    optimizer" page, sections 1.3 and 4) without printing any; the round itself
    is the same map."""
    if schedule is None:
        schedule = [(a, b, c)] * steps
    schedule = [tuple(float(v) for v in abc) for abc in schedule]
    u = np.asarray(u, dtype=np.float64)
    out = np.empty_like(u)
    for i in range(u.shape[0]):
        x = u[i]
        tall = x.shape[0] > x.shape[1]
        if tall:
            x = x.T
        x = frobenius_prescale(x, eps)
        for (ra, rb, rc) in schedule:
            gram = x @ x.T
            poly = rb * gram + rc * (gram @ gram)
            x = ra * x + poly @ x
        out[i] = x.T if tall else x
    return out


# ---------------------------------------------------------------------------
# mixed-precision apply
# ---------------------------------------------------------------------------

def recombine(hi, lo) -> np.ndarray:
    """fp32 master bits = (bf16 bits << 16) | low mantissa (Record 7 page, section 4.1)."""
    return (np.asarray(hi, dtype=np.uint16).astype(np.uint32) << np.uint32(16)) | \
        np.asarray(lo, dtype=np.uint16).astype(np.uint32)


def split(bits):
    """fp32 master bits -> (high half = new bf16 bits, low half = new mantissa):
    a bit slice, i.e. truncation (Record 7 page, section 4.1)."""
    bits = np.asarray(bits, dtype=np.uint32)
    return (bits >> np.uint32(16)).astype(np.uint16), (bits & np.uint32(0xFFFF)).astype(np.uint16)


def mp_apply_update(w_hi, w_lo, v, eta, decay: float):
    """w = fp32(hi, lo);  t = RN32(w * decay);  r = RN32(t - eta*v);  split(r).

    ``v`` holds bf16 values (float64 array), ``eta`` and ``decay`` are float32
    scalars or arrays broadcastable to v (one value per slot).
    The decay multiply comes before the update (Record 7 page, section 4.1).
    w*decay and eta*v are exact in float64 (<=48- and <=32-bit significands);
    t - eta*v is exact unless TwoSum reports an error, and those elements are
    rounded from exact rationals.  Finite weights only."""
    w = recombine(w_hi, w_lo).view(np.float32).astype(np.float64)
    v = np.asarray(v, dtype=np.float64)
    eta_b = np.broadcast_to(np.asarray(eta, dtype=np.float64), v.shape)
    t = round_to_f32(w * np.asarray(decay, dtype=np.float64))
    prod = eta_b * v
    s = t - prod
    bb = s - t
    err = (t - (s - bb)) + (-prod - bb)
    r = round_to_f32(s)
    p, emin, emax = _FORMATS[F32]
    for idx in zip(*np.nonzero((err != 0) & np.isfinite(s))):
        q = Fraction(float(t[idx])) - Fraction(float(eta_b[idx])) * Fraction(float(v[idx]))
        r[idx] = round_fraction(q, p, emin, emax)
    return split(r.astype(np.float32).view(np.uint32))


# ---------------------------------------------------------------------------
# the whole step
# ---------------------------------------------------------------------------

def muon_bank_step(grad, buf, w_hi, w_lo, storage: str, *, lr: float = 0.02,
                   weight_decay: float = 0.01, momentum: float = 0.95,
                   lr_mul: float = 1.0, wd_mul: float = 1.0, lr_mul_per_slot=None, slot_scalars=None,
                   steps: int = NS_STEPS, a: float = NS_COEFFS[0], b: float = NS_COEFFS[1],
                   c: float = NS_COEFFS[2], eps: float = NS_EPS, schedule=None) -> dict:
    """One Muon step on a viewed bank [batch, rows, cols].

    grad and buf are float64 arrays of values of the storage format (fp32 or
    bf16); w_hi/w_lo are the uint16 bf16 weight bits and low mantissas.  The
    defaults are Muon's constructor defaults lr=0.02, weight_decay=0.01,
    momentum=0.95 ("Muon Custom Sizing", section 2.2).  ``lr_mul_per_slot``
    (float32 values, one per slot) multiplies eta once more in float32.
    ``slot_scalars`` ([batch, 4] float32 values: mu, nu, decay, eta of each
    slot) replaces all of these per slot: every bank's momentum, decay and
    per-matrix learning rate held in one float32 table, as the "Unified
    zero-copy optimizer and transposed LM head" page, section 4, keeps them in
    one device buffer uploaded once per step.  Dead (all-zero) slots need no
    special case: every stage maps zero to zero."""
    grad = np.asarray(grad, dtype=np.float64)
    _, rows, cols = grad.shape
    sc = step_scalars(lr, weight_decay, momentum, rows, cols, lr_mul, wd_mul)
    if slot_scalars is not None:
        if lr_mul_per_slot is not None:
            raise ValueError("slot_scalars already holds each slot's eta")
        tab = np.asarray(slot_scalars, dtype=np.float64).reshape(grad.shape[0], 4)
        mu, nu, decay, eta = (tab[:, k][:, None, None] for k in range(4))
    else:
        mu, nu, decay = sc.mu, sc.nu, sc.decay
        if lr_mul_per_slot is None:
            eta = sc.eta
        else:
            per = np.asarray(lr_mul_per_slot, dtype=np.float64)
            eta = round_to_f32(sc.eta * per)[:, None, None]
    buf_new, u = momentum_nesterov(grad, buf, mu, nu, storage)
    v64 = newton_schulz(u, steps, a, b, c, eps, schedule=schedule)
    v = round_to_bf16(v64)
    hi, lo = mp_apply_update(w_hi, w_lo, v, eta, decay)
    return {"momentum": buf_new, "u": u, "v64": v64, "v": v, "w_hi": hi, "w_lo": lo,
            "scalars": sc, "eta": eta, "decay": decay}
