"""The pins have teeth: copies of the oracle with one planted mistake each must fail a pin.

Each mutant is the oracle source with one textual substitution, compiled on
the CPU into a temporary directory.  The planted mistakes live only in those
temporary copies; the oracle itself is never modified.
"""
import os
import subprocess

import pytest

import pins
from oracle import OracleLib
from oracle.oracle import SRC

MUTANTS = {
    "causal_off_by_one": ("if (causal && j > i) allowed = 0;", "if (causal && j >= i) allowed = 0;"),
    "causal_bottom_right": ("if (causal && j > i) allowed = 0;", "if (causal && j > i + (kL - qL)) allowed = 0;"),
    "gqa_wrong_kv_head": ("const int64_t g = h / group;", "const int64_t g = h % Hkv;"),
    "scale_dropped": ("double sc = scale * dot;", "double sc = dot;"),
    "mask_scaled_too": ("if (mask_kind == 1) sc = sc + mrow[j];", "if (mask_kind == 1) sc = scale * (dot + mrow[j]);"),
    "mask_sign": ("if (mask_kind == 1) sc = sc + mrow[j];", "if (mask_kind == 1) sc = sc - mrow[j];"),
    "bool_polarity": ("if (mask_kind == 2 && mrow[j] == 0.0) allowed = 0;",
                      "if (mask_kind == 2 && mrow[j] != 0.0) allowed = 0;"),
    "neg_inf_kept": ("if (sc == -INFINITY) allowed = 0;", ""),
    "dot_drops_last_term": ("for (int d = 0; d < D; ++d) dot += q[d] * k[d];",
                            "for (int d = 0; d < D - 1; ++d) dot += q[d] * k[d];"),
    "max_not_subtracted_from_L": ("*lse = m + log(l);", "*lse = log(l);"),
    "log2_instead_of_ln": ("*lse = m + log(l);", "*lse = m + log2(l);"),
    "no_normalisation": ("for (int d = 0; d < D; ++d) o[d] = o[d] / l;", ""),
    "v_is_k": ("const double* v = vbase + j * D;", "const double* v = kbase + j * D;"),
    "empty_row_L_neg_inf": ("*lse = 0.0;", "*lse = -INFINITY;"),
    "mask_row_ignores_head": ("mask + flat * (int64_t)kL", "mask + i * (int64_t)kL"),
    "row_max_wrong": ("if (s[j] > m) m = s[j];", "if (s[j] > m) m = s[j] * 0.5;"),
    "exp_of_negated": ("const double p = exp(s[j] - m);", "const double p = exp(m - s[j]);"),
    "query_head_index": ("const int64_t h = bh % Hq;", "const int64_t h = bh % Hkv;"),
}


def _build_mutant(tmpdir, name, old, new):
    with open(SRC) as f:
        src = f.read()
    assert src.count(old) == 1, f"mutant {name}: pattern must occur exactly once"
    path = os.path.join(tmpdir, f"{name}.c")
    with open(path, "w") as f:
        f.write(src.replace(old, new))
    so = os.path.join(tmpdir, f"lib_{name}.so")
    subprocess.run(["gcc", "-O1", "-fopenmp", "-shared", "-fPIC", "-std=c99", path, "-o", so, "-lm"], check=True)
    return so


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(tmp_path, name):
    old, new = MUTANTS[name]
    lib = OracleLib(_build_mutant(str(tmp_path), name, old, new))
    caught = []
    for pin in pins.ALL_PINS:
        try:
            pin(lib.fwd)
        except (AssertionError, ValueError, FloatingPointError):
            caught.append(pin.__name__)
    assert caught, f"no pin catches the planted mistake {name}"
