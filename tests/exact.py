"""Exact-arithmetic brute force used to pin the oracle (no GPU, no oracle code).

Means and variances are computed in exact rationals (``fractions.Fraction``
from the exact binary value of each fp32/fp64 input); square roots and
quotients in 60-digit ``decimal``.  Written from the definitions of the three
normalizations, independently of ``oracle/oracle.c``:

* LayerNorm (LN page "Kimi-K2.6 l1_p40", turn 1): per sample, population mean
  and variance over all normalized elements; (x - mean) / sqrt(var + eps),
  then elementwise weight and bias.
* GroupNorm -> LeakyReLU -> x + x (GN page "Kimi-K2.6 l2_p62", turn 1):
  contiguous groups of C/G channels, per-(row, group) population statistics,
  per-channel affine, LeakyReLU, doubling.
* RMSNorm along dim 1 (RMS page "Kimi-K2.6 l1_p36", turns 1-2):
  x / sqrt(mean over channels of x^2 + eps).
* fc -> GroupNorm -> LeakyReLU -> x + x (GN page, turn 1): h = x W^T + b as
  exact rationals, then the GroupNorm epilogue above on the exact h.
"""
from decimal import Decimal, getcontext
from fractions import Fraction

getcontext().prec = 60


def _dec(fr: Fraction) -> Decimal:
    return Decimal(fr.numerator) / Decimal(fr.denominator)


def _fr(v) -> Fraction:
    return Fraction(float(v))


def layer_norm(seg, w=None, b=None, eps=1e-5):
    """One segment (a flat list of numbers): returns (y list of Decimal, mean, var) exactly."""
    xs = [_fr(v) for v in seg]
    n = len(xs)
    mean = sum(xs, Fraction(0)) / n
    var = sum(((v - mean) ** 2 for v in xs), Fraction(0)) / n
    denom = _dec(var + _fr(eps)).sqrt()
    out = []
    for i, v in enumerate(xs):
        y = _dec(v - mean) / denom
        if w is not None:
            y = y * _dec(_fr(w[i]))
        if b is not None:
            y = y + _dec(_fr(b[i]))
        out.append(y)
    return out, mean, var


def group_norm_lrelu_x2(row, gamma, beta, G, eps, slope):
    """One row of C channels: returns the C outputs as Decimal."""
    C = len(row)
    M = C // G
    out = []
    for g in range(G):
        seg = row[g * M:(g + 1) * M]
        z, _, _ = layer_norm(seg, None, None, eps)
        for j in range(M):
            c = g * M + j
            v = z[j]
            if gamma is not None:
                v = v * _dec(_fr(gamma[c]))
            if beta is not None:
                v = v + _dec(_fr(beta[c]))
            a = v if v > 0 else _dec(_fr(slope)) * v
            out.append(a + a)
    return out


def rms_position(vals, eps):
    """The C values of one position: returns the C outputs as Decimal and the mean square."""
    xs = [_fr(v) for v in vals]
    ms = sum((v * v for v in xs), Fraction(0)) / len(xs)
    denom = _dec(ms + _fr(eps)).sqrt()
    return [_dec(v) / denom for v in xs], ms


def _group_epilogue(hs, gamma, beta, G, eps, slope):
    """GroupNorm -> LeakyReLU -> x + x of one row given as exact rationals."""
    C = len(hs)
    M = C // G
    out = []
    for g in range(G):
        seg = hs[g * M:(g + 1) * M]
        mean = sum(seg, Fraction(0)) / M
        var = sum(((v - mean) ** 2 for v in seg), Fraction(0)) / M
        denom = _dec(var + _fr(eps)).sqrt()
        for j in range(M):
            c = g * M + j
            v = _dec(seg[j] - mean) / denom
            if gamma is not None:
                v = v * _dec(_fr(gamma[c]))
            if beta is not None:
                v = v + _dec(_fr(beta[c]))
            a = v if v > 0 else _dec(_fr(slope)) * v
            out.append(a + a)
    return out


def fc_group_norm_lrelu_x2(x_row, W, bias, gamma, beta, G, eps, slope):
    """One row of x [K] through h = x W^T + b (W [C, K]), exact, then the GroupNorm epilogue: the C
    outputs as Decimal."""
    xs = [_fr(v) for v in x_row]
    hs = []
    for c in range(len(W)):
        acc = sum((xs[k] * _fr(W[c][k]) for k in range(len(xs))), Fraction(0))
        if bias is not None:
            acc += _fr(bias[c])
        hs.append(acc)
    return _group_epilogue(hs, gamma, beta, G, eps, slope)
