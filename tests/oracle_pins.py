"""Pins for the CPU oracle: checks against things other than the oracle itself.

Each ``pin_*`` function takes an ``oracle.Oracle`` instance and raises
AssertionError if the oracle disagrees with exact brute force, a closed form,
an invariant, a special case or an independent library routine.  The pins
run against the real oracle (tests/test_oracle_pins.py) and against builds
of oracle.c with a planted mistake (tests/test_oracle_mutants.py), which they
must reject.
"""
import numpy as np

from tests import exact

EPS32 = float(np.float32(1e-5))


def _close(got, want, tol):
    got = float(got)
    want = float(want)
    assert abs(got - want) <= tol * (1.0 + abs(want)), (got, want)


# ---------------------------------------------------------------- brute force

def pin_ln_bruteforce(orc, seed=0):
    """LayerNorm of tiny random segments == exact rationals (LN page, turn 1)."""
    rng = np.random.default_rng(seed)
    for outer, inner, eps, affine in [(1, 1, 1e-5, True), (2, 5, 1e-5, True), (3, 7, 0.25, True),
                                      (2, 12, 1e-5, False), (1, 9, 2.0, True)]:
        x = (rng.standard_normal((outer, inner)) * rng.uniform(0.1, 10) + rng.uniform(-5, 5))
        x = x.astype(np.float32)
        w = rng.standard_normal(inner).astype(np.float32) if affine else None
        b = rng.standard_normal(inner).astype(np.float32) if affine else None
        y, mean, var = orc.ln(x, w, b, eps=eps, return_stats=True)
        eps32 = float(np.float32(eps))
        for r in range(outer):
            ey, em, ev = exact.layer_norm(x[r], w, b, eps32)
            _close(mean[r], float(em), 1e-14)
            _close(var[r], float(ev), 1e-13)
            for i in range(inner):
                _close(y[r, i], float(ey[i]), 1e-12)


def pin_gn_bruteforce(orc, seed=1):
    """GroupNorm -> LeakyReLU -> x2 of tiny rows == exact rationals (GN page, turn 1)."""
    rng = np.random.default_rng(seed)
    for N, C, G, eps, slope in [(2, 8, 2, 1e-5, 0.01), (3, 12, 3, 0.1, 0.2), (2, 6, 1, 1e-5, 0.5),
                                (1, 10, 5, 1e-5, 0.01), (2, 16, 4, 1.0, 0.3)]:
        x = (rng.standard_normal((N, C)) * 2.0 - 0.5).astype(np.float32)
        gamma = (1.0 + 0.5 * rng.standard_normal(C)).astype(np.float32)
        beta = (0.5 * rng.standard_normal(C)).astype(np.float32)
        y = orc.gn_lrelu_x2(x, gamma, beta, G, eps=eps, negative_slope=slope)
        for n in range(N):
            ey = exact.group_norm_lrelu_x2(x[n], gamma, beta, G, float(np.float32(eps)),
                                           float(np.float32(slope)))
            for c in range(C):
                _close(y[n, c], float(ey[c]), 1e-12)
        assert (y < 0).any() and (y > 0).any()


def pin_rms_bruteforce(orc, seed=2):
    """RMSNorm along dim 1 of tiny tensors == exact rationals (RMS page, turns 1-2)."""
    rng = np.random.default_rng(seed)
    for shape, eps in [((2, 3, 5), 1e-5), ((1, 1, 4), 1e-5), ((2, 5, 2, 3), 0.5), ((3, 4, 1), 1e-5),
                       ((1, 7, 3), 3.0)]:
        x = (rng.standard_normal(shape) * rng.uniform(0.01, 3)).astype(np.float32)
        y, ms = orc.rms_ch(x, eps=eps, return_ms=True)
        B, C = shape[0], shape[1]
        S = int(np.prod(shape[2:]))
        xf = x.reshape(B, C, S)
        yf = y.reshape(B, C, S)
        for b in range(B):
            for s in range(S):
                ey, ems = exact.rms_position(xf[b, :, s], float(np.float32(eps)))
                _close(ms[b, s], float(ems), 1e-14)
                for c in range(C):
                    _close(yf[b, c, s], float(ey[c]), 1e-12)


def pin_fc_numpy(orc, seed=3):
    """fc == numpy's float64 matmul (an independent library routine), non-square W."""
    rng = np.random.default_rng(seed)
    for N, K, Cout in [(3, 5, 7), (4, 33, 6), (1, 64, 2), (3, 0, 5)]:  # K = 0: the empty sum, h = b
        x = rng.standard_normal((N, K)).astype(np.float32)
        W = rng.uniform(-1, 1, (Cout, K)).astype(np.float32)
        b = rng.uniform(-1, 1, Cout).astype(np.float32)
        h = orc.fc(x, W, b)
        want = x.astype(np.float64) @ W.astype(np.float64).T + b.astype(np.float64)
        np.testing.assert_allclose(h, want, rtol=1e-13, atol=1e-13)


def pin_fc_gn_bruteforce(orc, seed=10):
    """fc -> GroupNorm -> LeakyReLU -> x2 of tiny problems == exact rationals (GN page, turn 1).  eps and
    negative_slope differ enough that exchanging them changes the result, and the inputs carry enough
    bits that rounding h to fp32 before the GroupNorm would too."""
    rng = np.random.default_rng(seed)
    for N, K, C, G, eps, slope in [(2, 5, 8, 2, 0.3, 0.05), (1, 7, 6, 3, 1e-5, 0.2), (2, 3, 4, 1, 2.0, 0.01)]:
        x = (rng.standard_normal((N, K)) * 3.0).astype(np.float32)
        W = rng.uniform(-1, 1, (C, K)).astype(np.float32)
        b = (rng.uniform(-1, 1, C) + 20.0).astype(np.float32)
        gamma = (1.0 + 0.5 * rng.standard_normal(C)).astype(np.float32)
        beta = (0.5 * rng.standard_normal(C)).astype(np.float32)
        y = orc.fc_gn_lrelu_x2(x, W, b, gamma, beta, G, eps=eps, negative_slope=slope)
        for n in range(N):
            ey = exact.fc_group_norm_lrelu_x2(x[n], W, b, gamma, beta, G, float(np.float32(eps)),
                                              float(np.float32(slope)))
            for c in range(C):
                _close(y[n, c], float(ey[c]), 1e-12)
        assert (y < 0).any() and (y > 0).any()


# ------------------------------------------------------- closed forms, invariants

def pin_ln_closed_forms(orc, seed=4):
    """With weight 1 and bias 0: sum(y) = 0 and mean(y^2) = v / (v + eps) (LN page, turn 1)."""
    rng = np.random.default_rng(seed)
    for inner, eps in [(1000, 1e-5), (777, 0.3), (64, 5.0)]:
        x = (rng.standard_normal((2, inner)) * 0.7 + 3.0).astype(np.float32)
        y = orc.ln(x, eps=eps)
        xd = x.astype(np.float64)
        v = np.var(xd, axis=1)  # numpy's own variance (population, ddof=0)
        e = float(np.float32(eps))
        for r in range(2):
            assert abs(y[r].sum()) <= 1e-9 * inner
            _close(np.mean(y[r] ** 2), v[r] / (v[r] + e), 1e-11)


def pin_ln_special_cases(orc, seed=5):
    """One-element or constant segments give y = bias; eps=0 makes LN affine-invariant."""
    rng = np.random.default_rng(seed)
    b = rng.standard_normal(6).astype(np.float32)
    w = rng.standard_normal(6).astype(np.float32)
    const = np.full((2, 6), 3.25, np.float32)
    np.testing.assert_array_equal(orc.ln(const, w, b), np.broadcast_to(b.astype(np.float64), (2, 6)))
    one = rng.standard_normal((4, 1)).astype(np.float32)
    np.testing.assert_array_equal(orc.ln(one, w[:1], b[:1]), np.broadcast_to(b[:1].astype(np.float64), (4, 1)))
    # eps = 0: LN(a*x + c) = sign(a) * LN(x)
    x = rng.standard_normal((2, 50))
    y0 = orc.ln(x, eps=0.0)
    np.testing.assert_allclose(orc.ln(-3.0 * x + 7.0, eps=0.0), -y0, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(orc.ln(0.5 * x - 1.0, eps=0.0), y0, rtol=1e-12, atol=1e-12)
    # permutation equivariance
    perm = rng.permutation(50)
    np.testing.assert_allclose(orc.ln(x[:, perm], eps=1e-5), orc.ln(x, eps=1e-5)[:, perm],
                               rtol=1e-13, atol=1e-13)


def pin_ln_uniform_moments(orc, seed=6):
    """U[0,1) samples: mean -> 1/2 and variance -> 1/12 within 6 sigma (LN page, turn 2)."""
    rng = np.random.default_rng(seed)
    n = 1 << 20
    x = rng.random((1, n)).astype(np.float32)
    _, mean, var = orc.ln(x, return_stats=True)
    # std of the sample mean: sqrt(1/12/n); of the sample variance: sqrt((1/80 - 1/144)/n)
    assert abs(mean[0] - 0.5) < 6 * np.sqrt(1 / 12 / n)
    assert abs(var[0] - 1 / 12) < 6 * np.sqrt((1 / 80 - 1 / 144) / n)


def pin_ln_cancellation(orc, seed=7):
    """N(100, 0.01) data (large mean, tiny variance): the variance is exact to 1e-12 relative."""
    rng = np.random.default_rng(seed)
    x = (100.0 + 0.01 * rng.standard_normal((1, 10000))).astype(np.float32)
    _, mean, var = orc.ln(x, return_stats=True)
    _, em, ev = exact.layer_norm(x[0], None, None, EPS32)
    assert abs(mean[0] - float(em)) <= 1e-13 * abs(float(em))
    assert abs(var[0] - float(ev)) <= 1e-12 * float(ev)


def pin_gn_special_cases(orc, seed=8):
    """GN with one channel per group gives 2*lrelu(beta); GN with one group is LayerNorm of the row."""
    rng = np.random.default_rng(seed)
    N, C = 3, 12
    x = rng.standard_normal((N, C)).astype(np.float32)
    gamma = (1 + 0.3 * rng.standard_normal(C)).astype(np.float32)
    beta = rng.standard_normal(C).astype(np.float32)
    slope = float(np.float32(0.01))
    bd = beta.astype(np.float64)
    want = 2.0 * np.where(bd > 0, bd, slope * bd)
    np.testing.assert_array_equal(orc.gn_lrelu_x2(x, gamma, beta, C, negative_slope=0.01),
                                  np.broadcast_to(want, (N, C)))
    # G = 1: the group is the whole row; statistics from numpy, affine + epilogue written out here
    y = orc.gn_lrelu_x2(x, gamma, beta, 1, eps=1e-5, negative_slope=0.01)
    xd = x.astype(np.float64)
    mu = xd.mean(axis=1, keepdims=True)
    v = xd.var(axis=1, keepdims=True)
    z = (xd - mu) / np.sqrt(v + EPS32) * gamma.astype(np.float64) + bd
    np.testing.assert_allclose(y, 2.0 * np.where(z > 0, z, slope * z), rtol=1e-12, atol=1e-12)
    # closed form per group with identity affine: sum = 0 over a group before the epilogue is
    # not observable after LeakyReLU, so check instead that gamma=1, beta=0, slope=1 gives
    # 2 * normalized values, whose per-group mean square is v/(v+eps)
    G = 3
    y = orc.gn_lrelu_x2(x, None, None, G, eps=1e-5, negative_slope=1.0) / 2.0
    for n in range(N):
        for g in range(G):
            seg = xd[n, g * 4:(g + 1) * 4]
            vg = seg.var()
            _close(np.mean(y[n, g * 4:(g + 1) * 4] ** 2), vg / (vg + EPS32), 1e-12)
            assert abs(y[n, g * 4:(g + 1) * 4].sum()) < 1e-12


def pin_rms_closed_forms(orc, seed=9):
    """RMS: C = 1 gives x / sqrt(x^2 + eps); mean over channels of y^2 = ms / (ms + eps)."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((3, 1, 17)).astype(np.float32)
    xd = x.astype(np.float64)
    np.testing.assert_allclose(orc.rms_ch(x), xd / np.sqrt(xd * xd + EPS32), rtol=1e-14, atol=0)
    x = rng.standard_normal((2, 9, 4, 5)).astype(np.float32)
    y = orc.rms_ch(x)
    ms = np.mean(x.astype(np.float64) ** 2, axis=1)
    np.testing.assert_allclose(np.mean(y ** 2, axis=1), ms / (ms + EPS32), rtol=1e-12)
    # scaling: rms_ch(a x) with eps scaled by a^2 equals rms_ch(x) (eps values exact in fp32)
    np.testing.assert_allclose(orc.rms_ch(4.0 * x, eps=4.0), orc.rms_ch(x, eps=0.25), rtol=1e-13)


ALL_PINS = [
    pin_ln_bruteforce, pin_gn_bruteforce, pin_rms_bruteforce, pin_fc_numpy, pin_fc_gn_bruteforce,
    pin_ln_closed_forms, pin_ln_special_cases, pin_ln_uniform_moments, pin_ln_cancellation,
    pin_gn_special_cases, pin_rms_closed_forms,
]
