"""Planted mistakes in the oracle, each caught by a pin (CPU only).

Every case edits the oracle's source, one mistake per case (a dropped term, a transposed operand, a wrong norm,
a missing round, swapped coefficients, a rounding where the pages slice bits, a rounding too many or too few, ...),
executes the edited functions in a copy of the oracle's namespace, binds them where a pin test looks them up,
and runs that pin: it must fail.  The unedited oracle passes the same pins in tests/test_oracle_*.py.  A case whose
source line is no longer in the oracle fails too, so an edit of the oracle cannot silently retire a case.

One plausible mistake is not on the list because no pin can catch it: working on a tall slot without
transposing it gives the same result in exact arithmetic (p(X^T) = p(X)^T), only with the larger Gram.
"""

import inspect

import pytest

import oracle.muon as om
import oracle.transpose as ot
from tests import (test_oracle_apply, test_oracle_momentum, test_oracle_ns, test_oracle_rounding, test_oracle_step,
                   test_oracle_transpose)


def mutant(edits, rebuild):
    """Namespace copy of the oracle module that defines the edited functions (oracle.muon or
    oracle.transpose) in which `edits` [(function, old line text, new text)] are applied and every
    function in `rebuild` is re-executed, so that they call the edited ones."""
    names = list(dict.fromkeys([e[0] for e in edits] + list(rebuild)))
    mod = om if hasattr(om, names[0]) else ot
    ns = dict(mod.__dict__)
    for name in names:
        src = inspect.getsource(getattr(mod, name))
        for fn, old, new in edits:
            if fn == name:
                assert old in src, f"{name}: the line to edit is gone from the oracle: {old!r}"
                src = src.replace(old, new)
        exec(compile(src, f"<mutant {name}>", "exec"), ns)
    return ns


# (case id, edits, functions to re-execute, {pin module: names to rebind}, pin test, its arguments)
CASES = [
    ("ns drops the c*A*A term",
     [("newton_schulz", "poly = rb * gram + rc * (gram @ gram)", "poly = rb * gram")], [],
     {test_oracle_ns: ["newton_schulz"]}, test_oracle_ns.test_ns_equals_svd_closed_form, ((8, 8),)),
    ("ns Gram of the transpose",
     [("newton_schulz", "gram = x @ x.T", "gram = x.T @ x")], [],
     {test_oracle_ns: ["newton_schulz"]}, test_oracle_ns.test_ns_equals_svd_closed_form, ((8, 8),)),
    ("ns update subtracts B X",
     [("newton_schulz", "x = ra * x + poly @ x", "x = ra * x - poly @ x")], [],
     {test_oracle_ns: ["newton_schulz"]}, test_oracle_ns.test_ns_equals_svd_closed_form, ((4, 16),)),
    ("ns one round short",
     [("newton_schulz", "for (ra, rb, rc) in schedule:", "for (ra, rb, rc) in schedule[:-1]:")], [],
     {test_oracle_ns: ["newton_schulz"]}, test_oracle_ns.test_ns_equals_svd_closed_form, ((6, 12),)),
    ("ns spectral norm instead of Frobenius",
     [("frobenius_prescale", "return x / (math.sqrt(float(np.sum(x * x))) + eps)",
       "return x / (float(np.linalg.norm(x, 2)) + eps)")], ["newton_schulz"],
     {test_oracle_ns: ["newton_schulz", "frobenius_prescale"]}, test_oracle_ns.test_ns_equals_svd_closed_form,
     ((16, 4),)),
    ("momentum swaps mu and nu",
     [("momentum_nesterov", "buf_new = _round_sum_of_products(mu, buf, nu, grad, storage)",
       "buf_new = _round_sum_of_products(nu, buf, mu, grad, storage)")], [],
     {test_oracle_momentum: ["momentum_nesterov"]}, test_oracle_momentum.test_momentum_is_exactly_rounded_bf16, ()),
    ("u from the unrounded buffer",
     [("momentum_nesterov", "u = _round_sum_of_products(nu, grad, mu, buf_new, BF16)",
       "u = _round_sum_of_products(nu, grad, mu, np.asarray(mu) * np.asarray(buf) + np.asarray(nu) * "
       "np.asarray(grad), BF16)")], [],
     {test_oracle_momentum: ["momentum_nesterov"]}, test_oracle_momentum.test_momentum_is_exactly_rounded_bf16, ()),
    ("bf16 rounding truncates",
     [("round_to_format", "y = np.rint(x / quantum) * quantum", "y = np.trunc(x / quantum) * quantum")],
     ["round_to_bf16"],
     {test_oracle_rounding: ["round_to_bf16"]}, test_oracle_rounding.test_bf16_rounding_matches_brute_force_search,
     ()),
    ("the split rounds instead of slicing",
     [("split", "return (bits >> np.uint32(16)).astype(np.uint16), (bits & np.uint32(0xFFFF)).astype(np.uint16)",
       "return ((bits + np.uint32(0x8000)) >> np.uint32(16)).astype(np.uint16), "
       "(bits & np.uint32(0xFFFF)).astype(np.uint16)")], [],
     {test_oracle_apply: ["split"]}, test_oracle_apply.test_split_is_a_bit_slice, ()),
    ("the apply drops the decay",
     [("mp_apply_update", "t = round_to_f32(w * np.asarray(decay, dtype=np.float64))", "t = w")], [],
     {test_oracle_apply: ["mp_apply_update"]}, test_oracle_apply.test_apply_is_exactly_rounded_on_random_inputs, ()),
    ("per-slot eta not rounded to float32",
     [("muon_bank_step", "eta = round_to_f32(sc.eta * per)[:, None, None]", "eta = (sc.eta * per)[:, None, None]")],
     [], {test_oracle_step: ["muon_bank_step"]}, test_oracle_step.test_per_slot_eta_is_one_fp32_multiply, ()),
    ("transpose_copy reverses the row order",
     [("transpose_copy", "out[:, i] = src[i, :]", "out[:, i] = src[rows - 1 - i, :]")], [],
     {test_oracle_transpose: ["transpose_copy"]}, test_oracle_transpose.test_copy_is_the_transpose_by_brute_force_and_numpy,
     ()),
    ("transpose_add reshapes src instead of transposing it",
     [("transpose_add", "src_t = transpose_copy(src)", "src_t = np.asarray(src).reshape(dst.shape)")], [],
     {test_oracle_transpose: ["transpose_add"]}, test_oracle_transpose.test_add_f32_is_the_correctly_rounded_sum, ()),
    ("transpose_add leaves the float32 sum unrounded",
     [("transpose_add", "return round_to_f32(s).astype(np.float32)", "return s")], [],
     {test_oracle_transpose: ["transpose_add"]}, test_oracle_transpose.test_add_f32_is_the_correctly_rounded_sum, ()),
    ("the apply rounds eta*v before subtracting it",
     [("mp_apply_update", "prod = eta_b * v", "prod = round_to_f32(eta_b * v)")], [],
     {test_oracle_apply: ["mp_apply_update"]}, test_oracle_apply.test_apply_is_exactly_rounded_on_random_inputs, ()),
    ("recombine swaps the two halves",
     [("recombine", "np.asarray(hi,", "np.asarray(HALF,"), ("recombine", "np.asarray(lo,", "np.asarray(hi,"),
      ("recombine", "np.asarray(HALF,", "np.asarray(lo,")], ["mp_apply_update"],
     {test_oracle_apply: ["mp_apply_update"]}, test_oracle_apply.test_apply_identities, ()),
    ("nu is one minus the rounded mu",
     [("step_scalars", "nu=_f32(1.0 - momentum),", "nu=_f32(1.0 - _f32(momentum)),")], [],
     {test_oracle_momentum: ["step_scalars"]}, test_oracle_momentum.test_step_scalars_closed_forms, ()),
    ("a float32 buffer is stored as bf16",
     [("momentum_nesterov", "buf_new = _round_sum_of_products(mu, buf, nu, grad, storage)",
       "buf_new = _round_sum_of_products(mu, buf, nu, grad, BF16)")], [],
     {test_oracle_momentum: ["momentum_nesterov"]}, test_oracle_momentum.test_momentum_is_exactly_rounded_fp32, ()),
    ("eps under the square root of the norm",
     [("frobenius_prescale", "return x / (math.sqrt(float(np.sum(x * x))) + eps)",
       "return x / math.sqrt(float(np.sum(x * x)) + eps)")], ["newton_schulz"],
     {test_oracle_ns: ["newton_schulz", "frobenius_prescale"]}, test_oracle_ns.test_ns_equals_svd_closed_form,
     ((8, 8),)),
    ("a schedule runs its rounds in reverse",
     [("newton_schulz", "for (ra, rb, rc) in schedule:", "for (ra, rb, rc) in schedule[::-1]:")], [],
     {test_oracle_ns: ["newton_schulz"]}, test_oracle_ns.test_schedule_equals_composed_closed_form, ((6, 12),)),
    ("float32 rounding without gradual underflow",
     [("round_to_format", "ex = np.maximum(e.astype(np.int64) - 1, emin)", "ex = e.astype(np.int64) - 1")],
     ["round_to_f32"], {test_oracle_rounding: ["round_to_f32"]}, test_oracle_rounding.test_f32_rounding_matches_numpy_cast,
     ()),
    ("step reads u from the unrounded buffer",
     [("momentum_nesterov", "u = _round_sum_of_products(nu, grad, mu, buf_new, BF16)",
       "u = _round_sum_of_products(nu, grad, mu, np.asarray(mu) * np.asarray(buf) + np.asarray(nu) * "
       "np.asarray(grad), BF16)")], ["muon_bank_step"],
     {test_oracle_step: ["muon_bank_step"]}, test_oracle_step.test_nesterov_reads_the_stored_buffer, ()),
]


@pytest.mark.filterwarnings("ignore::RuntimeWarning")
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_pin_catches_planted_mistake(case, monkeypatch):
    _, edits, rebuild, bind, pin, args = case
    ns = mutant(edits, rebuild)
    for module, names in bind.items():
        for name in names:
            monkeypatch.setattr(module, name, ns[name])
    with pytest.raises(AssertionError):
        pin(*args)


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_the_unedited_oracle_passes_the_same_pin(case):
    """Control: the pin passes with the oracle as it is (re-executed the same way, with no edit)."""
    _, edits, rebuild, bind, pin, args = case
    ns = mutant([], [e[0] for e in edits] + list(rebuild))
    with pytest.MonkeyPatch.context() as mp:
        for module, names in bind.items():
            for name in names:
                mp.setattr(module, name, ns[name])
        pin(*args)
