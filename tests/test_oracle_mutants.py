"""Planted mistakes in the oracle are caught by its pins.

Each case compiles a copy of oracle.c with one plausible mistake (a dropped
term, a wrong scale, a wrong index or order) and runs every pin in
test_oracle_pins.py against it; at least one pin must fail.  Everything runs on
the CPU in temporary files; the real oracle is untouched.
"""
import inspect
import os

import pytest

from oracle import oracle as _o
from tests import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(_o.__file__), "oracle.c")

MUTANTS = {
    "scale 1/d instead of 1/sqrt(d)": ("1.0 / sqrt((double)d)", "1.0 / (double)d"),
    "alpha without the log": ("*alpha = M + log(Z);", "*alpha = M + Z;"),
    "GQA head taken modulo": ("int h = hq / G;", "int h = hq % Hkv;"),
    "ties go to the higher index": ("return x->pos < y->pos ? -1 : 1;", "return x->pos > y->pos ? -1 : 1;"),
    "sink window one short": ("i < n && i < n_sink;", "i < n && i < n_sink - 1;"),
    "recent window one short": ("(n - n_recent > 0 ? n - n_recent : 0)", "(n - n_recent + 1 > 0 ? n - n_recent + 1 : 0)"),
    "merge drops e^alpha from the denominator": ("double Z = w_doc;", "double Z = 0.0;"),
    "popcount skips the top bit": ("bit < 32", "bit < 31"),
    "bf16 expanded with the wrong shift": ("(uint32_t)bits << 16", "(uint32_t)bits << 15"),
    "value row read reversed": ("out[c] += w * elem(v, dtype, kv_off + j * d + c);",
                                "out[c] += w * elem(v, dtype, kv_off + j * d + (d - 1 - c));"),
    "batch stride ignored": ("(int64_t)b * kv_batch_stride", "(int64_t)0 * kv_batch_stride"),
    "local value rows not used": ("o[c] += w * elem(v_loc, dtype, kv_off + i * d + c);",
                                  "o[c] += w * elem(v_loc, dtype, kv_off + c);"),
    "signature of a zero projection set": ("if (z > 0.0) c |= 1u << b;", "if (z >= 0.0) c |= 1u << b;"),
    "signature bits reversed": ("if (z > 0.0) c |= 1u << b;", "if (z > 0.0) c |= 1u << (bits - 1 - b);"),
    "projection read transposed": ("(double)R[(int64_t)e * bits + b]", "(double)R[(int64_t)b * d + e]"),
    "wide codes skip the last word": ("for (int w = 0; w < W; ++w) dist +=", "for (int w = 0; w < W - 1; ++w) dist +="),
    "wide codes read one word per key": ("hamming32(ks[i * W + w], qw[w])", "hamming32(ks[i + w], qw[w])"),
}


def _pin_tests():
    out = []
    for name, fn in inspect.getmembers(pins, inspect.isfunction):
        if name.startswith("test_") and "orc" in inspect.signature(fn).parameters:
            out.append(fn)
    return out


def _run(fn, orc):
    kw = {"orc": orc}
    if "n" in inspect.signature(fn).parameters:
        kw["n"] = 7
    if "W" in inspect.signature(fn).parameters:
        kw["W"] = 4
    fn(**kw)


def test_real_oracle_passes_every_pin():
    orc = _o.default()
    for fn in _pin_tests():
        _run(fn, orc)


@pytest.mark.parametrize("label", sorted(MUTANTS))
def test_mutant_is_caught(label, tmp_path):
    old, new = MUTANTS[label]
    src = open(SRC).read()
    assert old in src, "mutation site not found: %r" % old
    mut = tmp_path / "oracle_mutant.c"
    mut.write_text(src.replace(old, new))
    (tmp_path / "oracle.h").write_text(open(SRC.replace(".c", ".h")).read())
    lib = _o.build(force=True, src=str(mut), out=str(tmp_path / "libmut.so"))
    orc = _o.Oracle(lib)
    failed = []
    for fn in _pin_tests():
        try:
            _run(fn, orc)
        except (AssertionError, ValueError) as e:  # a pin rejected the mutant
            failed.append(fn.__name__)
    assert failed, "no pin caught the planted mistake: " + label
