"""The pins are strong enough: plausible mistakes planted in a copy of the oracle's C source (a
dropped term, a wrong sign, index or alignment, the wrong head or row) are each caught by at least one
of the oracle's pins.  Every mutant is a one-line change of oracle/cqsa_oracle.c built with gcc into a
temporary library that the oracle package loads in place of its own for the duration of the test;
the pins then run unchanged (the same functions as tests/test_oracle_pins.py and
tests/test_oracle_backward_pins.py).  Every mutant keeps all its accesses in bounds."""
import ctypes
import functools
import subprocess

import pytest
import torch

import oracle
import test_oracle_backward_pins as BP
import test_oracle_pins as P

FORWARD_MUTANTS = [
    ("top-left causal alignment", "int64_t last = i + (p->Nk - p->Nq); /* last visible key */",
     "int64_t last = i; /* last visible key */"),
    ("diagonal key masked", "if (hi > last + 1) hi = last + 1;", "if (hi > last) hi = last;"),
    ("GQA head by modulo", "const int64_t hk = h / g;\n        /* visible keys", "const int64_t hk = h % p->Hkv;\n        /* visible keys"),
    ("scale dropped", "s[j - lo] = sigma * dot;", "s[j - lo] = dot;"),
    ("exponent sign flipped", "const double w = exp(s[j - lo] - m);", "const double w = exp(m - s[j - lo]);"),
    ("lse without the shift", "m + log(l) : -INFINITY;", "log(l) : -INFINITY;"),
    ("query rows reversed", "h * p->q_stride[1] + i * p->q_stride[2]);\n        for",
     "h * p->q_stride[1] + (p->Nq - 1 - i) * p->q_stride[2]);\n        for"),
    ("values from head 0", "hk * p->v_stride[1] + j * p->v_stride[2]);\n            for (int64_t t = 0; t < D; ++t) nsum",
     "0 * p->v_stride[1] + j * p->v_stride[2]);\n            for (int64_t t = 0; t < D; ++t) nsum"),
    ("output not normalised", "(osum[t] + ocomp[t]) / l : NAN;", "(osum[t] + ocomp[t]) : NAN;"),
    ("merge: l without weights", "l[r] = alpha * a_l + beta * b_l;", "l[r] = a_l + b_l;"),
    ("merge: second weight from the first m", "exp(b_m - mm);", "exp(a_m - mm);"),
    ("fp16 exponent bias", "e - 25); /* (1024 + f)", "e - 24); /* (1024 + f)"),
]

BACKWARD_MUTANTS = [
    ("dS sign", "const double ds = P * (dP - st[2]);", "const double ds = P * (st[2] - dP);"),
    ("dQ without the scale", "dq[t] += sigma * ds *", "dq[t] += ds *"),
    ("row term D_i unweighted", "Di += exp(s[j] - m) / l * dp[j];", "Di += dp[j];"),
    ("dK/dV skip the diagonal row",
     "i0 = j - (p->Nk - p->Nq) > 0 ? j - (p->Nk - p->Nq) : 0;",
     "i0 = j - (p->Nk - p->Nq) + 1 > 0 ? j - (p->Nk - p->Nq) + 1 : 0;"),
    ("GQA gradients from one head", "for (int64_t h = hk * g; h < (hk + 1) * g; ++h) {",
     "for (int64_t h = hk * g; h < hk * g + 1; ++h) {"),
    ("dV with unnormalised P", "const double P = exp(sij - st[0]) / st[1];", "const double P = exp(sij - st[0]);"),
]

_SHAPES = [(1, 1, 1, 1, 1, 1), (1, 2, 1, 5, 7, 3), (2, 4, 2, 8, 8, 4), (1, 3, 3, 3, 6, 2)]
FORWARD_PINS = (
    [("fp16 decode", P.test_fp16_decode_every_bit_pattern), ("bf16 decode", P.test_bf16_decode_every_bit_pattern)]
    + [(f"golden {d}", functools.partial(P.test_golden_worked_examples, d)) for d in (torch.float16, torch.bfloat16)]
    + [(f"brute force {c} {s}", functools.partial(P.test_bruteforce_longdouble, c, s))
       for c in (False, True) for s in _SHAPES]
    + [(f"sdpa {c}", functools.partial(P.test_matches_torch_sdpa_float64, torch.float16, c))
       for c in ("noncausal_rect", "causal_square", "gqa_causal", "gqa_noncausal")]
    + [("weights sum to one", functools.partial(P.test_weights_sum_to_one, True)),
       ("causal row 0", functools.partial(P.test_causal_row0_is_v0, torch.float16)),
       ("q = 0 closed form", functools.partial(P.test_q_zero_closed_form, 5, 23)),
       ("bottom-right offset", P.test_bottom_right_is_tail_of_square),
       ("GQA = MHA", P.test_gqa_equals_mha_on_repeated_kv),
       ("constant v, single key", P.test_constant_v_and_single_key),
       ("zero scale", P.test_zero_scale_gives_uniform_weights),
       ("key permutation", P.test_noncausal_key_permutation_invariance),
       ("identity partial", P.test_identity_partial_and_merge_identity)]
    + [(f"split invariance {c} {t}", functools.partial(P.test_any_split_merged_equals_unsplit, c, t))
       for c in (False, True) for t in range(2)]
    + [("partial normalises", P.test_partial_normalises_to_full)]
)
BACKWARD_PINS = (
    [(f"autograd {a}", functools.partial(BP.test_backward_matches_float64_autograd, *a))
     for a in [(1, 2, 2, 7, 7, True, 4, torch.float16), (1, 4, 2, 5, 9, True, 3, torch.bfloat16),
               (2, 2, 1, 6, 4, False, 5, torch.float16)]]
    + [("finite differences", BP.test_backward_matches_finite_differences_of_the_forward),
       ("closed forms and invariants", BP.test_closed_forms_and_invariants),
       ("GQA gradients = MHA", BP.test_gqa_gradients_equal_mha_on_repeated_kv)]
)


def _build_mutant(tmp_path, old: str, new: str) -> str:
    src = open(oracle._SRC).read()
    assert src.count(old) == 1, f"mutation site not unique or missing: {old!r}"
    path = tmp_path / "mutant.c"
    path.write_text(src.replace(old, new))
    lib = tmp_path / "libmutant.so"
    subprocess.check_call(["gcc", *oracle.CFLAGS, "-o", str(lib), str(path), "-lm"])
    return str(lib)


def _catches(pins) -> list:
    """Names of the pins that fail."""
    failed = []
    for name, pin in pins:
        try:
            pin()
        except (AssertionError, ValueError, RuntimeError):   # a failed check, or values the check rejects
            failed.append(name)
    return failed


def _run(tmp_path, monkeypatch, old, new, pins):
    monkeypatch.setattr(oracle, "_LIB_PATH", _build_mutant(tmp_path, old, new))
    monkeypatch.setattr(oracle, "_lib", None)
    return _catches(pins)


def test_pins_pass_on_the_unmutated_oracle(tmp_path, monkeypatch):
    """The harness itself: the same build route with no change passes every pin."""
    anchor = "const double sigma = (double)p->scale;\n    const int64_t g"
    assert _run(tmp_path, monkeypatch, anchor, anchor, FORWARD_PINS + BACKWARD_PINS) == []


@pytest.mark.parametrize("name,old,new", FORWARD_MUTANTS, ids=[m[0] for m in FORWARD_MUTANTS])
def test_forward_pins_catch_mutant(name, old, new, tmp_path, monkeypatch):
    caught = _run(tmp_path, monkeypatch, old, new, FORWARD_PINS)
    assert caught, f"no pin caught the mutant: {name}"
    print(f"{name}: caught by {len(caught)} pins: {caught}")


@pytest.mark.parametrize("name,old,new", BACKWARD_MUTANTS, ids=[m[0] for m in BACKWARD_MUTANTS])
def test_backward_pins_catch_mutant(name, old, new, tmp_path, monkeypatch):
    caught = _run(tmp_path, monkeypatch, old, new, BACKWARD_PINS)
    assert caught, f"no pin caught the mutant: {name}"
    print(f"{name}: caught by {len(caught)} pins: {caught}")


def test_the_real_oracle_is_restored():
    """After the mutants, the package's own library is the one loaded (monkeypatch undoes the swap)."""
    lib = oracle._load()
    assert isinstance(lib, ctypes.CDLL) and lib._name == oracle._LIB_PATH
    P.test_causal_row0_is_v0(torch.float16)
