"""The oracle's pins are meant to catch any plausible slip in it.  This checks
that claim on the CPU: copies of the oracle's C source, each with one planted
mistake, are compiled into a temporary directory and run through the pins of
``test_oracle_pins.py``; every mutant must fail at least one pin, and the
unmodified source, built the same way, must pass all of them.

Every mutant keeps its memory accesses inside the caller's buffers (a wrong
leading dimension is replaced by a smaller one, a wrong index by a mirrored
one), so a mutant can give wrong values but never fault.
"""
import importlib.util
import os
import shutil

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
ORACLE_PY = os.path.join(ROOT, "oracle", "oracle.py")
ORACLE_C = os.path.join(ROOT, "oracle", "oracle_sgemm.c")

# name -> (text in oracle_sgemm.c, replacement); each text occurs exactly once.
MUTANTS = {
    "alpha dropped": ("(double)alpha * acc[j]", "acc[j]"),
    "beta term dropped": ("(double)alpha * acc[j] + (double)beta * (double)C[i * ldc + j]",
                          "(double)alpha * acc[j]"),
    "beta term subtracted": ("acc[j] + (double)beta", "acc[j] - (double)beta"),
    "alpha and beta swapped": ("(double)alpha * acc[j] + (double)beta * (double)C",
                               "(double)beta * acc[j] + (double)alpha * (double)C"),
    "first k term dropped": ("for (int64_t k = 0; k < K; ++k) {\n        const double a",
                             "for (int64_t k = 1; k < K; ++k) {\n        const double a"),
    "last k term dropped": ("for (int64_t k = 0; k < K; ++k) {\n        const double a",
                            "for (int64_t k = 0; k < K - 1; ++k) {\n        const double a"),
    "B row shifted": ("const float *brow = B + k * ldb;",
                      "const float *brow = B + ((k + 1) % K) * ldb;"),
    "B column mirrored": ("acc[j] += a * (double)brow[j];", "acc[j] += a * (double)brow[N - 1 - j];"),
    "lda taken as K": ("(double)A[i * lda + k];\n        const float *brow",
                       "(double)A[i * K + k];\n        const float *brow"),
    "ldb taken as N": ("const float *brow = B + k * ldb;", "const float *brow = B + k * N;"),
    "ldc taken as N on store": ("C[i * ldc + j] = (float)v;", "C[i * N + j] = (float)v;"),
    "products rounded to fp32": ("acc[j] += a * (double)brow[j];",
                                 "acc[j] += (float)(a * (double)brow[j]);"),
    "entries: B column mirrored": ("s += (double)A[i * lda + k] * (double)B[k * ldb + j];",
                                   "s += (double)A[i * lda + k] * (double)B[k * ldb + (N - 1 - j)];"),
    "entries: beta term dropped": ("const double v = (double)alpha * s + (double)beta * (double)Cin[i * ldc + j];",
                                   "const double v = (double)alpha * s;"),
}


def _load_pins():
    spec = importlib.util.spec_from_file_location("oracle_pins_for_mutants",
                                                  os.path.join(HERE, "test_oracle_pins.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _pin_calls(pins):
    """Every pin once, with the first value set of its parametrisation."""
    calls = []
    for name in sorted(dir(pins)):
        f = getattr(pins, name)
        if not (name.startswith("test_") and callable(f)):
            continue
        kwargs = {}
        for mark in getattr(f, "pytestmark", []):
            if mark.name == "parametrize":
                names = [n.strip() for n in mark.args[0].split(",")]
                first = list(mark.args[1])[0]
                kwargs.update(zip(names, first if len(names) > 1 else (first,)))
        calls.append((name, f, kwargs))
    return calls


def _build_variant(src_text, where, tag):
    """A copy of oracle.py whose library is built from `src_text` in `where`."""
    spec = importlib.util.spec_from_file_location(f"oracle_variant_{tag}", ORACLE_PY)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    os.makedirs(where, exist_ok=True)
    mod.SRC = os.path.join(where, "oracle_sgemm.c")
    mod.LIB = os.path.join(where, "liboracle_sgemm.so")
    mod._lib = None
    with open(mod.SRC, "w") as f:
        f.write(src_text)
    mod.build(force=True)
    return mod


def _failing_pins(mod, calls):
    failed = []
    for name, f, kwargs in calls:
        try:
            f(mod, **kwargs)
        except Exception:  # an assertion, or an error status from the mutant
            failed.append(name)
    return failed


@pytest.fixture(scope="module")
def pins_and_source(tmp_path_factory):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    return _pin_calls(_load_pins()), open(ORACLE_C).read(), tmp_path_factory.mktemp("oracle_mutants")


def test_unmodified_source_passes_every_pin(pins_and_source):
    calls, src, tmp = pins_and_source
    mod = _build_variant(src, os.path.join(tmp, "original"), "original")
    assert _failing_pins(mod, calls) == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_every_planted_mistake_fails_a_pin(pins_and_source, name):
    calls, src, tmp = pins_and_source
    old, new = MUTANTS[name]
    assert src.count(old) == 1, f"mutation site for {name!r} not unique in the oracle source"
    tag = "".join(ch if ch.isalnum() else "_" for ch in name)
    mod = _build_variant(src.replace(old, new), os.path.join(tmp, tag), tag)
    assert _failing_pins(mod, calls), f"no pin detects: {name}"
