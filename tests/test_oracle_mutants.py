"""Planted mistakes in copies of the oracle (CPU only; test infrastructure).

Each mutant is `oracle/mqa_oracle.c` with one plausible slip planted by text
substitution in a temporary copy, compiled with gcc the way the oracle is.
Every mutant must fail at least one of the oracle's pins (exact brute force,
hand-worked golden files, the fp8 table from torch's conversion, the hoist and
paged-gather invariants), and the unchanged copy must pass all of them: the
pins pin the oracle, not just agree with it.
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import pytest

import oracle
from tests import test_oracle as pins

SRC = os.path.join(os.path.dirname(os.path.abspath(oracle.__file__)), "mqa_oracle.c")

_BOUND = "int64_t bound = (int64_t)ctx[b] - next_n + j; /* inclusive */"
MUTANTS = {
    "dropped relu": ("double r = dot > 0.0 ? dot : 0.0; /* relu */", "double r = dot; /* relu */"),
    "prefill window end inclusive": ("if (n >= lo && n < hi)", "if (n >= lo && n <= hi)"),
    "prefill window start exclusive": ("if (n >= lo && n < hi)", "if (n > lo && n < hi)"),
    "decode bound one short": (_BOUND, _BOUND.replace("+ j;", "+ j - 1;")),
    "decode bound one long": (_BOUND, _BOUND.replace("+ j;", "+ j + 1;")),
    "wrong gather slot": ("int64_t slot = p % bs;", "int64_t slot = (p + 1) % bs;"),
    "wrong scale slot": ("memcpy(&sc, base + (int64_t)bs * D + slot * 4, 4);",
                         "memcpy(&sc, base + (int64_t)bs * D + ((slot + 1) % bs) * 4, 4);"),
    "shifted weight index": ("acc += r * scale * (double)w[h];",
                             "acc += r * scale * (double)w[(h + 1) % H];"),
    "transposed Q": ("dot += table_fp8[q[(int64_t)h * D + d]] * table_fp8[k[d]];",
                     "dot += table_fp8[q[(int64_t)d * H + h]] * table_fp8[k[d]];"),
    "hoisted scale dropped": ("return hoist ? acc * scale : acc;", "return acc;"),
    "exponent bias 8": ("v = ldexp(1.0 + (double)m / 8.0, e - 7);",
                        "v = ldexp(1.0 + (double)m / 8.0, e - 8);"),
    "subnormal exponent": ("v = ldexp((double)m / 8.0, 1 - 7);", "v = ldexp((double)m / 8.0, -7);"),
}


def _params(func):
    """The argument tuples of a parametrized test function."""
    for mark in getattr(func, "pytestmark", []):
        if mark.name == "parametrize":
            return [v if isinstance(v, tuple) else (v,) for v in mark.args[1]]
    return [()]


def _pins():
    """(name, callable) for the pins, cheapest first."""
    out = [("fp8 table", pins.test_fp8_table_matches_torch_conversion),
           ("hand example", pins.test_hand_example_prefill_and_decode),
           ("hoist", pins.test_hoisted_scale_equals_unhoisted)]
    out += [("windows %s" % (c[:2],), lambda c=c: pins.test_golden_windows(c))
            for c in pins._golden_windows()]
    out += [("prefill brute %s" % (a,), lambda a=a: pins.test_prefill_matches_exact_brute_force(*a))
            for a in _params(pins.test_prefill_matches_exact_brute_force)]
    out += [("decode brute %s" % (a,), lambda a=a: pins.test_decode_matches_exact_brute_force(*a))
            for a in _params(pins.test_decode_matches_exact_brute_force)]
    out += [("paged = contiguous D%d" % a, lambda a=a: pins.test_paged_decode_equals_contiguous_prefill(*a))
            for a in _params(pins.test_paged_decode_equals_contiguous_prefill)]
    return out


def _build(tmp_path, name, subst):
    text = open(SRC).read()
    if subst is not None:
        old, new = subst
        assert text.count(old) == 1, "mutation site not found: %s" % name
        text = text.replace(old, new)
    tag = name.replace(" ", "_")
    src = tmp_path / ("%s.c" % tag)
    lib = tmp_path / ("lib%s.so" % tag)
    src.write_text(text)
    subprocess.check_call(["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared", "-o", str(lib),
                           str(src), "-lm"])
    so = ctypes.CDLL(str(lib))
    P, i32, i64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
    so.oracle_e4m3fn_value.restype = ctypes.c_double
    so.oracle_e4m3fn_value.argtypes = [ctypes.c_uint8]
    so.oracle_e4m3fn_table.argtypes = [P]
    so.oracle_num_threads.restype = i32
    so.oracle_set_num_threads.argtypes = [i32]
    so.oracle_prefill.argtypes = [P, P, P, P, P, P, i64, i64, i32, i32, i32, i32, P]
    so.oracle_decode.restype = i32
    so.oracle_decode.argtypes = [P, P, P, P, P, i32, i32, i32, i32, i32, i32, i64, i32, i64, i32,
                                 i32, P]
    return so


def _failing_pins(monkeypatch, so, stop_at_first):
    monkeypatch.setattr(oracle, "_lib", so)
    failed = []
    for name, pin in _pins():
        try:
            pin()
        except Exception as e:  # an assertion or an oracle error: the pin caught the slip
            failed.append("%s: %s" % (name, type(e).__name__))
            if stop_at_first:
                break
    return failed


def test_unchanged_copy_passes_every_pin(tmp_path, monkeypatch):
    assert _failing_pins(monkeypatch, _build(tmp_path, "unchanged", None), False) == []


@pytest.mark.parametrize("name", list(MUTANTS))
def test_planted_mistake_fails_a_pin(tmp_path, monkeypatch, name):
    failed = _failing_pins(monkeypatch, _build(tmp_path, name, MUTANTS[name]), True)
    assert failed, "no pin caught the planted mistake: %s" % name
