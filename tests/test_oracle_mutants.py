"""Planted mistakes in copies of the oracle (CPU only; test infrastructure).

Each mutant is one oracle source with one plausible slip planted by text
substitution: `oracle/mqa_oracle.c` in a temporary copy compiled with gcc the
way the oracle is, or the top-k and K-cache modules executed from their edited
text.  Every mutant must fail at least one of that oracle's pins (exact brute
force, hand-worked golden files, the fp8 table from torch's conversion, the
hoist and paged-gather invariants, the pairwise top-k rule, torch's fp8
rounding), and the unchanged copy must pass all of them: the pins pin the
oracle, not just agree with it.
"""

from __future__ import annotations

import ctypes
import functools
import inspect
import os
import subprocess
import types

import pytest

import oracle
from oracle import kcache, topk
from tests import test_oracle as pins
from tests import test_oracle_kcache as kcache_pins
from tests import test_oracle_topk as topk_pins

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


# ---- the Python oracles: top-k order and K-cache quantise/insert ----

_PY_MUTANTS = {
    "topk ties by larger column": (topk, topk_pins, "np.lexsort((cols, -v[cols]))",
                                   "np.lexsort((-cols, -v[cols]))"),
    "topk ascending": (topk, topk_pins, "np.lexsort((cols, -v[cols]))", "np.lexsort((cols, v[cols]))"),
    "topk -inf listable": (topk, topk_pins, "(v == -np.inf)", "(v == np.inf)"),
    "topk NaN listable": (topk, topk_pins, "~(np.isnan(v) | (v == -np.inf))", "~(v == -np.inf)"),
    "topk padding 0": (topk, topk_pins, "np.full((rows, k), -1,", "np.full((rows, k), 0,"),
    "topk one short": (topk, topk_pins, "[:k]", "[:max(k - 1, 1)]"),
    "kcache scale over 256": (kcache, kcache_pins, "/ np.float32(FP8_MAX)).astype", "/ np.float32(256.0)).astype"),
    "kcache signed amax": (kcache, kcache_pins, "amax = np.abs(k).max(axis=-1)", "amax = k.max(axis=-1)"),
    "kcache epsilon": (kcache, kcache_pins, "np.float32(1e-12)", "np.float32(1e-6)"),
    "kcache ties to odd": (kcache, kcache_pins, "codes[lo] % 2 == 0", "codes[lo] % 2 == 1"),
    "kcache truncation": (kcache, kcache_pins, "pick = np.where(d_lo < d_hi, lo, hi)", "pick = lo"),
    "kcache sign dropped": (kcache, kcache_pins, "np.where(np.signbit(v.ravel()), out | 0x80, out)",
                            "np.where(np.signbit(v.ravel()), out, out)"),
    "kcache scale slot": (kcache, kcache_pins, "off = block_size * D + 4 * slot",
                          "off = block_size * D + 4 * ((slot + 1) % block_size)"),
    "kcache tile stride": (kcache, kcache_pins, "(d // 16) * 256", "(d // 16) * 128"),
    "kcache padding written": (kcache, kcache_pins, "if s < 0 or", "if s < -1 or"),
    "kcache last slot written": (kcache, kcache_pins, "s >= num_slots:", "s > num_slots:"),
}


def _cases(module):
    """(name, call) for every test function of a pin module, each
    parametrization expanded (stacked decorators give the product)."""
    out = []
    for name, f in vars(module).items():
        if not name.startswith("test_") or not callable(f):
            continue
        grids = [{}]
        for mark in getattr(f, "pytestmark", []):
            if mark.name != "parametrize":
                continue
            names = mark.args[0]
            names = [n.strip() for n in names.split(",")] if isinstance(names, str) else list(names)
            grids = [{**g, **dict(zip(names, v if len(names) > 1 else (v,)))}
                     for g in grids for v in mark.args[1]]
        params = set(inspect.signature(f).parameters)
        assert all(set(g) == params for g in grids), "pin %s needs a fixture" % name
        out += [("%s %s" % (name, g), functools.partial(f, **g)) for g in grids]
    return out


def _mutant_module(mod, subst):
    text = inspect.getsource(mod)
    if subst is not None:
        old, new = subst
        assert text.count(old) == 1, "mutation site not found: %r" % old
        text = text.replace(old, new)
    m = types.ModuleType(mod.__name__ + "_mutant")
    m.__file__ = mod.__file__
    exec(compile(text, mod.__file__, "exec"), m.__dict__)
    return m


def _patch(monkeypatch, pin_module, orig, mutant):
    """Point every name of the pin module that refers to the oracle module, or
    to one of its functions, at the mutant's."""
    for name, val in list(vars(pin_module).items()):
        if val is orig:
            monkeypatch.setattr(pin_module, name, mutant)
        elif inspect.isfunction(val) and val.__module__ == orig.__name__:
            monkeypatch.setattr(pin_module, name, getattr(mutant, val.__name__))


def _failing_py_pins(monkeypatch, orig, pin_module, subst, stop_at_first):
    _patch(monkeypatch, pin_module, orig, _mutant_module(orig, subst))
    failed = []
    for name, pin in _cases(pin_module):
        try:
            pin()
        except Exception as e:  # an assertion or an oracle error: the pin caught the slip
            failed.append("%s: %s" % (name, type(e).__name__))
            if stop_at_first:
                break
    return failed


@pytest.mark.parametrize("orig,pin_module", [(topk, topk_pins), (kcache, kcache_pins)],
                         ids=["topk", "kcache"])
def test_unchanged_python_oracle_passes_every_pin(monkeypatch, orig, pin_module):
    assert _failing_py_pins(monkeypatch, orig, pin_module, None, False) == []


@pytest.mark.parametrize("name", list(_PY_MUTANTS))
def test_planted_python_mistake_fails_a_pin(monkeypatch, name):
    orig, pin_module, old, new = _PY_MUTANTS[name]
    failed = _failing_py_pins(monkeypatch, orig, pin_module, (old, new), True)
    assert failed, "no pin caught the planted mistake: %s" % name
