"""The stored small cases: the oracle reproduces them, and the first LayerNorm row
matches its closed form (x = 1..8: mean 9/2, population variance 21/4)."""
import json
import os
from decimal import Decimal, getcontext

import numpy as np

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))


def _cases():
    with open(os.path.join(HERE, "golden", "small_cases.json")) as f:
        return json.load(f)["cases"]


def _arr(v):
    return None if v is None else np.array(v, np.float32)


def test_oracle_reproduces_golden():
    for c in _cases():
        want = np.array(c["y"], dtype=object).astype(np.float64)
        if c["op"] == "ln":
            got = oracle.ln(_arr(c["x"]), _arr(c["weight"]), _arr(c["bias"]), eps=c["eps"])
        elif c["op"] == "gn_lrelu_x2":
            got = oracle.gn_lrelu_x2(_arr(c["x"]), _arr(c["gamma"]), _arr(c["beta"]),
                                     c["num_groups"], eps=c["eps"],
                                     negative_slope=c["negative_slope"])
        else:
            got = oracle.rms_ch(_arr(c["x"]), eps=c["eps"])
        np.testing.assert_array_equal(got, want, err_msg=c["cite"])


def test_golden_ln_row_closed_form():
    """LN page, turn 1: y = (x - mean)/sqrt(var + eps)*w + b with mean 4.5 and var 5.25 for 1..8."""
    getcontext().prec = 50
    c = _cases()[0]
    eps = Decimal(float(np.float32(c["eps"])))
    denom = (Decimal("5.25") + eps).sqrt()
    for i in range(8):
        xi = Decimal(i + 1)
        want = (xi - Decimal("4.5")) / denom * Decimal(c["weight"][i]) + Decimal(c["bias"][i])
        assert abs(float(c["y"][0][i]) - float(want)) <= 1e-15 * (1 + abs(float(want)))
