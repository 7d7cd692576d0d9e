"""Write tests/golden/small_cases.json: tiny hand-chosen inputs and the oracle's outputs.

Calls only the oracle (oracle/).  The inputs are short lists of numbers that
are exact in fp32; the outputs are the oracle's unrounded float64 values,
stored with repr() so they round-trip exactly.  Each case names the page
passage that defines the operation:
  LN page  "Kimi-K2.6 l1_p40", turn 1   LayerNorm, population variance, eps in the root
  GN page  "Kimi-K2.6 l2_p62", turn 1   contiguous groups, LeakyReLU, x + x
  RMS page "Kimi-K2.6 l1_p36", turns 1-2  x / sqrt(mean_c x^2 + eps)
Run: python tests/golden/make_golden.py
"""
import json
import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__)))))
import oracle  # noqa: E402

HERE = os.path.dirname(os.path.abspath(__file__))


def main():
    cases = []
    x = np.array([[1.0, 2.0, 3.0, 4.0, 5.0, 6.0, 7.0, 8.0],
                  [0.5, -0.25, 8.0, -3.0, 0.125, 2.0, -1.5, 6.0]], np.float32)
    w = np.array([1.0, 0.5, -1.0, 2.0, 1.0, 0.25, 1.5, -0.5], np.float32)
    b = np.array([0.0, 0.25, -0.5, 1.0, 0.0, -1.0, 0.125, 0.5], np.float32)
    cases.append({"op": "ln", "cite": "LN page Kimi-K2.6 l1_p40, turn 1", "eps": 1e-5,
                  "x": x.tolist(), "weight": w.tolist(), "bias": b.tolist(),
                  "y": [[repr(float(v)) for v in r] for r in oracle.ln(x, w, b, eps=1e-5)]})
    cases.append({"op": "ln", "cite": "LN page Kimi-K2.6 l1_p40, turn 1 (eps large enough to matter)",
                  "eps": 0.5, "x": x.tolist(), "weight": None, "bias": None,
                  "y": [[repr(float(v)) for v in r] for r in oracle.ln(x, eps=0.5)]})
    gx = np.array([[1.0, -2.0, 3.0, -4.0, 0.5, 0.25, -0.75, 1.0],
                   [-1.0, -1.5, -2.0, 4.0, 2.0, 2.0, 2.0, 2.5]], np.float32)
    gamma = np.array([1.0, 2.0, 0.5, 1.0, -1.0, 1.0, 1.0, 0.5], np.float32)
    beta = np.array([0.0, 0.5, -0.5, 0.0, 0.25, 0.0, -1.0, 0.0], np.float32)
    cases.append({"op": "gn_lrelu_x2", "cite": "GN page Kimi-K2.6 l2_p62, turn 1", "num_groups": 2,
                  "eps": 1e-5, "negative_slope": 0.01, "x": gx.tolist(), "gamma": gamma.tolist(),
                  "beta": beta.tolist(),
                  "y": [[repr(float(v)) for v in r] for r in oracle.gn_lrelu_x2(gx, gamma, beta, 2)]})
    rx = np.array([[[1.0, -2.0, 0.5], [3.0, 0.0, -0.5], [-1.0, 2.0, 4.0]]], np.float32)
    cases.append({"op": "rms_ch", "cite": "RMS page Kimi-K2.6 l1_p36, turns 1-2", "eps": 1e-5,
                  "x": rx.tolist(),
                  "y": [[[repr(float(v)) for v in r] for r in p] for p in oracle.rms_ch(rx)]})
    with open(os.path.join(HERE, "small_cases.json"), "w") as f:
        json.dump({"generated_by": "tests/golden/make_golden.py (oracle only)", "cases": cases}, f)


if __name__ == "__main__":
    main()
