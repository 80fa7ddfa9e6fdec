"""Plain CPU oracle for the Muon bank step.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
load this package: only the test suite, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, table or
helper with the HIP library; both sides receive the same host arrays from
the seeded input generators and nothing else.

Everything is NumPy in float64 (plus ``fractions.Fraction`` where an exact
rounding decision needs more than 53 bits).  Each function cites the passage
of the pages it follows.  The pages are cited by title and section:

* "Unified zero-copy optimizer and transposed LM head" -- the walkthrough of
  the 2026-01-18 UnifiedOptimizers record; section 1.1 "Stacking vs.
  sharding: parameter banks" gives the bank shapes and the dead slot.
* "Muon Custom Sizing" -- the walkthrough of the 2025-09-23 MuonCustomSizing
  record; section 1 defines Muon, section 2.3 the batched Newton-Schulz
  call and its coefficients, section 4 the momentum lerps and the effective
  learning rate and weight decay.
* "GPT-2 Medium 25.29-minute record" -- the walkthrough of track-2 Record 7;
  section 4.1 gives the bf16 + uint16 mantissa apply, section 4.2 the five
  quintic iterations.
* "Unified zero-copy optimizer and transposed LM head", section 2.2, also
  gives the two tied-embedding transposes (``oracle/transpose.py``).
* "U-Net skips and doubled LR" -- the walkthrough of the 2024-11-10 record;
  its "four optimizers" section gives backend_steps=5, nesterov and the
  max(1, rows/cols)**0.5 scale.

Parity pins: every function here is pinned by ``tests/test_oracle_*.py``
against closed forms, library routines or exact rational arithmetic.  The
bf16 bits that a bf16 Newton-Schulz produces on a GPU depend on summation
order, so they are not pinned bit-for-bit: the NS comparison is a tolerance
(relative Frobenius error per slot), and the oracle's own NS is pinned to
the SVD closed form instead.
"""

from .muon import (  # noqa: F401
    BF16,
    F32,
    StepScalars,
    bf16_bits_to_f64,
    f64_to_bf16_bits,
    frobenius_prescale,
    momentum_nesterov,
    mp_apply_update,
    muon_bank_step,
    newton_schulz,
    recombine,
    round_fraction,
    round_to_bf16,
    round_to_f32,
    step_scalars,
    split,
)
from .transpose import transpose_add, transpose_copy  # noqa: F401
