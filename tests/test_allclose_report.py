"""The comparison every parity test uses (oracle.allclose_report) against its definition: an element
passes iff g is finite and |g - o| <= atol + rtol |o|, the bound taken relative to the oracle's value o
(not to g); max_rel is over |o| > 1e-3; n_bad counts the failing elements."""
import numpy as np
import pytest

import oracle


@pytest.mark.filterwarnings("ignore::RuntimeWarning")
def test_non_finite_values_fail_even_where_the_oracle_agrees():
    o = np.array([1.0, np.inf, -np.inf, 0.0])
    for g in ([np.nan, np.inf, -np.inf, 0.0], [1.0, np.inf, 0.0, 0.0], [1.0, 0.0, 0.0, np.nan]):
        rep = oracle.allclose_report(np.array(g), o, 1e-4, 1e-4)
        assert not rep["ok"]
    rep = oracle.allclose_report(np.array([np.nan, 1.0]), np.array([0.0, 1.0]), 1e-4, 1e-4)
    assert rep["n_bad"] == 1 and rep["worst_index"] == 0


def test_bound_is_atol_plus_rtol_times_the_oracle_value():
    atol, rtol = 1e-4, 1e-4
    o = np.array([0.0, 1.0, -50.0, 1e4])
    lim = atol + rtol * np.abs(o)
    assert oracle.allclose_report(o + 0.999 * lim, o, atol, rtol)["ok"]
    assert oracle.allclose_report(o - 0.999 * lim, o, atol, rtol)["ok"]
    for i in range(len(o)):  # one element just over its bound fails, alone
        g = o.copy()
        g[i] += 1.001 * lim[i]
        rep = oracle.allclose_report(g, o, atol, rtol)
        assert not rep["ok"] and rep["n_bad"] == 1 and rep["worst_index"] == i
    # relative to |o|, not |g|: at o = 1e4 an error of 1.00015 exceeds 1e-4 + 1e-4 * 1e4 = 1.0001,
    # though it would be within a bound taken from |g| = 10001.00015
    rep = oracle.allclose_report(np.array([1e4 + 1.00015]), np.array([1e4]), atol, rtol)
    assert not rep["ok"]
    # and at o = 0 only atol applies, however large g is relative to it
    assert not oracle.allclose_report(np.array([1.5e-4]), np.array([0.0]), atol, rtol)["ok"]


def test_reported_magnitudes():
    o = np.array([2.0, 1e-4, -4.0])
    g = np.array([2.002, 1e-4 + 5e-5, -4.0])
    rep = oracle.allclose_report(g, o, 1e-4, 1e-4)
    assert rep["n"] == 3 and rep["n_bad"] == 1 and rep["worst_index"] == 0
    assert rep["max_abs"] == pytest.approx(0.002)
    assert rep["max_rel"] == pytest.approx(0.001)  # over |o| > 1e-3 only: the 1e-4 entry is left out
    with pytest.raises(AssertionError):
        oracle.allclose_report(np.zeros(3), np.zeros(4), 1e-4, 1e-4)
