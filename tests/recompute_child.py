"""Run in a child process by test_gpu_recompute.py with NORMFWD_LN_FORCE_RECOMPUTE set (read once by the
library): the control-wave LayerNorm kernel then ignores the published sums of every k-th workgroup and
computes them from x itself, the path it takes when a workgroup is not resident.  Writes each output, its
statistics and the workspace's recompute count to an .npz file named on the command line."""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402
import torch  # noqa: E402

import normalization_ln_forward_amd as nf  # noqa: E402
from normalization_ln_forward_amd import synth  # noqa: E402

# (outer, inner, seed, workload): 3 workgroups per sample with a ragged last row, 32, 62 with a ragged last
# row, and 256 (every lane of the gather busy, stores interleaved with the next sample's loads) on the
# N(100, 0.01) stress input, with the 8 x 8 tile; 237 with a ragged last row with the wide 11 x 6 tile
CASES = [(5, 40000, 11, "ln_16x64x256x256"), (4, 1 << 19, 12, "ln_16x64x256x256"),
         (9, 1000004, 14, "ln_16x64x256x256"), (3, 1 << 22, 13, "ln_stress_16x64x256x256"),
         (8, 4000000, 15, "ln_16x64x256x256")]


# variant 1 (the tagged exchange) and variant 2 (last workgroup merges; not in place, so an ordinary launch
# in which a sample no merger announces is merged by whoever waited for it)
VARIANTS = (1, 2)


def run_cases():
    out = {}
    for (outer, inner, seed, name), variant in [(c, v) for c in CASES for v in VARIANTS]:
        d = synth.make(name, device="cuda", shape=(outer, inner), normalized_ndim=1, seed=seed)
        _, ws = nf.alloc_workspace(nf.ln_forward_workspace_size(outer, inner), "cuda")
        nf.ln_forward_workspace_init(ws)
        mean = torch.empty(outer, device="cuda")
        rstd = torch.empty(outer, device="cuda")
        y = nf.ln_forward(d["x"], d["weight"], d["bias"], variant=variant, workspace=ws, mean_out=mean,
                          rstd_out=rstd)
        if (outer, inner) == CASES[0][:2] and variant == 1:
            # past the 255-launch cycle of the exchange tags: words that are never accepted stay so
            for _ in range(300):
                again = nf.ln_forward(d["x"], d["weight"], d["bias"], variant=1, workspace=ws)
                if not torch.equal(again, y):
                    sys.exit("a repeated launch on one workspace changed the result")
        torch.cuda.synchronize()
        tag = f"v{variant}_{outer}x{inner}"
        out[f"y_{tag}"] = y.cpu().numpy()
        out[f"mean_{tag}"] = mean.cpu().numpy()
        out[f"rstd_{tag}"] = rstd.cpu().numpy()
        out[f"recomputed_{tag}"] = np.array(ws[:16].view(torch.int32).cpu().numpy()[3])
        print(f"{tag}: recomputed {int(out[f'recomputed_{tag}'])}", flush=True)
    return out


if __name__ == "__main__":
    np.savez(sys.argv[1], **run_cases())
    print("recompute child: ok", flush=True)
