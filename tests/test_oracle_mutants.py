"""Plant plausible mistakes in copies of oracle.c and check the pins reject every one.

Each mutant is a textual edit of the oracle source (a dropped term, a wrong
sign, a wrong divisor or index, a transposed operand), compiled into a
temporary library with the oracle's own flags.  A mutant passes this test
only if at least one pin from tests/oracle_pins.py fails on it, which shows
the pins are strong enough to catch that class of error in the real oracle.
"""
import os
import subprocess

import pytest

import oracle
from oracle import build as obuild
from tests import oracle_pins

MUTANTS = {
    # LayerNorm
    "ln_unbiased_var": ("const double var = ssd / (double)inner;",
                        "const double var = ssd / (double)(inner > 1 ? inner - 1 : 1);"),
    "ln_eps_outside_sqrt": ("const double denom = sqrt(var + eps);\n        if (mean_out) mean_out[r]",
                            "const double denom = sqrt(var) + eps;\n        if (mean_out) mean_out[r]"),
    "ln_bias_sign": ("if (b) v = v + b[i];", "if (b) v = v - b[i];"),
    "ln_weight_index": ("if (w) v = v * w[i];", "if (w) v = v * w[inner - 1 - i];"),
    "ln_mean_divisor": ("const double mean = sum / (double)inner;",
                        "const double mean = sum / (double)(inner + 1);"),
    # GroupNorm + LeakyReLU + x2
    "gn_interleaved_affine": ("const int64_t c = g * M + j;", "const int64_t c = j * G + g;"),
    "gn_slope_sign": ("const double a = z > 0.0 ? z : slope * z;",
                      "const double a = z > 0.0 ? z : -slope * z;"),
    "gn_no_double": ("y[n * C + c] = a + a;", "y[n * C + c] = a;"),
    "gn_unbiased_var": ("const double var = ssd / (double)M;",
                        "const double var = ssd / (double)(M > 1 ? M - 1 : 1);"),
    "gn_relu_instead_of_leaky": ("const double a = z > 0.0 ? z : slope * z;",
                                 "const double a = z > 0.0 ? z : 0.0;"),
    # RMSNorm
    "rms_sum_not_mean": ("const double ms = sumsq / (double)C;", "const double ms = sumsq;"),
    "rms_multiply": ("yp[c * S] = xp[c * S] / rms;", "yp[c * S] = xp[c * S] * rms;"),
    "rms_no_eps": ("const double rms = sqrt(ms + eps);", "const double rms = sqrt(ms);"),
    # fc
    "fc_transposed_W": ("acc += xr[k] * wr[k];", "acc += xr[k] * W[k * Cout + c];"),
    "fc_no_bias": ("if (bias) acc += bias[c];", "(void)bias;"),
}


def _build_mutant(tmpdir, name, old, new):
    src = open(obuild.SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not unique/found"
    path_c = os.path.join(tmpdir, f"{name}.c")
    path_so = os.path.join(tmpdir, f"{name}.so")
    with open(path_c, "w") as f:
        f.write(src.replace(old, new))
    subprocess.run(["gcc", *[fl for fl in obuild.CFLAGS if fl != "-Werror"], path_c, "-o",
                    path_so, "-lm"], check=True)
    return path_so


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_reject_mutant(name, tmp_path):
    old, new = MUTANTS[name]
    orc = oracle.Oracle(_build_mutant(str(tmp_path), name, old, new))
    failures = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(orc)
        except AssertionError:
            failures.append(pin.__name__)
    assert failures, f"no pin caught mutant {name}"


# The fc -> GroupNorm composition lives in oracle/__init__.py (Python), so its mutants are subclasses of
# the oracle that compose the two C functions the wrong way.
class _SwappedEpsSlope(oracle.Oracle):
    def fc_gn_lrelu_x2(self, x, W, bias, gamma, beta, num_groups, eps=1e-5, negative_slope=0.01):
        return self.gn_lrelu_x2(self.fc(x, W, bias), gamma, beta, num_groups, negative_slope, eps)


class _RoundedH(oracle.Oracle):
    def fc_gn_lrelu_x2(self, x, W, bias, gamma, beta, num_groups, eps=1e-5, negative_slope=0.01):
        h = self.fc(x, W, bias).astype("float32")
        return self.gn_lrelu_x2(h, gamma, beta, num_groups, eps, negative_slope)


class _GroupSizeForCount(oracle.Oracle):
    def fc_gn_lrelu_x2(self, x, W, bias, gamma, beta, num_groups, eps=1e-5, negative_slope=0.01):
        h = self.fc(x, W, bias)
        return self.gn_lrelu_x2(h, gamma, beta, h.shape[1] // num_groups, eps, negative_slope)


class _NoBias(oracle.Oracle):
    def fc_gn_lrelu_x2(self, x, W, bias, gamma, beta, num_groups, eps=1e-5, negative_slope=0.01):
        return self.gn_lrelu_x2(self.fc(x, W, None), gamma, beta, num_groups, eps, negative_slope)


@pytest.mark.parametrize("cls", [_SwappedEpsSlope, _RoundedH, _GroupSizeForCount, _NoBias],
                         ids=lambda c: c.__name__)
def test_fc_gn_pin_rejects_composition_mutant(cls):
    orc = cls(obuild.LIB if os.path.exists(obuild.LIB) else obuild.build())
    with pytest.raises(AssertionError):
        oracle_pins.pin_fc_gn_bruteforce(orc)
