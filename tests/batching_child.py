"""Run in a child process by test_gpu_batching.py with NORMFWD_MAX_GRID_ITEMS set low, so that every
launcher splits its grid into several launches of whole samples/rows; checks each result against the
oracle and exits non-zero on the first mismatch."""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import torch  # noqa: E402

import normalization_ln_forward_amd as nf  # noqa: E402
import oracle  # noqa: E402
from normalization_ln_forward_amd import synth  # noqa: E402


def check(name, got, ref, rtol=1e-4):
    rep = oracle.allclose_report(got.detach().cpu().numpy(), ref, atol=1e-4, rtol=rtol)
    print(f"{name}: {rep}", flush=True)
    if not rep["ok"]:
        sys.exit(1)


def main():
    assert os.environ.get("NORMFWD_MAX_GRID_ITEMS"), "run with NORMFWD_MAX_GRID_ITEMS set"
    npy = lambda t: t.detach().cpu().numpy()  # noqa: E731
    # LayerNorm: short samples (one workgroup each), the one-row normalize, the sample-loop normalize
    # (too big for one launch here, so it falls back to batched one-row launches), scalar and vector paths
    for outer, inner in ((700, 1000), (700, 1001), (20, 40000), (20, 40001), (3, 1 << 20), (2, (1 << 20) + 3)):
        d = synth.make("ln_16x64x256x256", device="cuda", shape=(outer, inner), normalized_ndim=1,
                       seed=outer + inner)
        mean = torch.empty(outer, device="cuda")
        rstd = torch.empty(outer, device="cuda")
        y = nf.ln_forward(d["x"], d["weight"], d["bias"], mean_out=mean, rstd_out=rstd)
        x64 = npy(d["x"]).astype("float64")
        check(f"ln {outer}x{inner}", y, oracle.ln(npy(d["x"]), npy(d["weight"]), npy(d["bias"])))
        check(f"ln mean {outer}x{inner}", mean, x64.mean(axis=1), rtol=1e-5)
    # GroupNorm: fast kernel (M = 16), lane kernel (M = 3), wave kernel (M = 100)
    for n, c, g in ((5000, 256, 16), (3000, 96, 32), (900, 1000, 10)):
        d = synth.make("gn_lrelu_x2_1024x8192", device="cuda", shape=(n, c), seed=n + c)
        y = nf.gn_lrelu_x2_forward(d["x"], d["gamma"], d["beta"], g)
        check(f"gn {n}x{c} G={g}", y, oracle.gn_lrelu_x2(npy(d["x"]), npy(d["gamma"]), npy(d["beta"]), g))
    # RMSNorm: register-held kernel and the streaming kernel for C > 512
    for b, c, s in ((40, 64, 4096), (40, 600, 2048)):
        d = synth.make("rms_ch_112x64x512x512", device="cuda", shape=(b, c, s), seed=b + c + s)
        check(f"rms {b}x{c}x{s}", nf.rmsnorm_ch_forward(d["x"]), oracle.rms_ch(npy(d["x"])))
    print("batching: ok", flush=True)


if __name__ == "__main__":
    main()
