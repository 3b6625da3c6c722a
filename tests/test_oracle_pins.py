"""The fp64 oracle against closed forms, invariants, brute force and torch (CPU only)."""
import json
import math
import os

import numpy as np
import pytest

import pins
from oracle import OracleLib, build_oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


@pytest.fixture(scope="module")
def oracle():
    build_oracle()
    return OracleLib()


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(oracle, pin):
    pin(oracle.fwd)


def test_golden_worked_examples(oracle):
    """Hand-derived worked examples whose expected values are closed forms (tests/golden)."""
    with open(os.path.join(GOLDEN, "worked_examples.json")) as f:
        cases = json.load(f)["cases"]
    env = {"e": math.e, "exp": math.exp, "log": math.log, "sqrt": math.sqrt, "inf": math.inf}
    for c in cases:
        q = np.array(c["q"], dtype=np.float64)[None, None]
        k = np.array(c["k"], dtype=np.float64)[None, None]
        v = np.array(c["v"], dtype=np.float64)[None, None]
        mask = None
        kind = c.get("mask_kind", "none")
        if kind != "none":
            mask = np.array([[eval(str(x), env) for x in row] for row in c["mask"]], dtype=np.float64)[None, None]
        O, L = oracle.fwd(q, k, v, scale=c["scale"], causal=c.get("causal", False), mask=mask, mask_kind=kind)
        expO = np.array([[eval(x, env) for x in row] for row in c["expect_O"]])
        expL = np.array([eval(x, env) for x in c["expect_L"]])
        np.testing.assert_allclose(O[0, 0], expO, rtol=0, atol=1e-13, err_msg=c["name"])
        np.testing.assert_allclose(L[0, 0], expL, rtol=0, atol=1e-13, err_msg=c["name"])


def test_rejects_bad_arguments(oracle):
    z = np.zeros((1, 3, 2, 4))
    kv = np.zeros((1, 2, 2, 4))
    with pytest.raises(ValueError):
        oracle.fwd(z, kv, kv, scale=1.0)  # 3 query heads over 2 kv heads
    with pytest.raises(ValueError):
        oracle.fwd(z, z, z, scale=1.0, rows=np.array([99]))
