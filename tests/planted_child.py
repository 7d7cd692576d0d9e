"""Run in a child process by test_gpu_numerics.py with NORMFWD_LN_FORCE_RECOMPUTE=4 (read once by the
library: every 4th workgroup of the single-read LayerNorm kernel publishes nothing, so its exchange slots
keep whatever other writers left there).  For each generation value: plant split-schedule partials in
every slot (a variant-0 call on the same workspace), set the control-wave generation word, run variant 1.
Writes the outputs and the recompute count to the .npz file named on the command line."""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402
import torch  # noqa: E402

import normalization_ln_forward_amd as nf  # noqa: E402
from normalization_ln_forward_amd import synth  # noqa: E402

SHAPE = (4, 1 << 19)  # 32 workgroups per sample in both the split and the single-read layout
# generation words: the range the kernel keeps it in, its ends, and values a workspace that was not zeroed
# could hold (the kernel reduces them mod 255); -1 is 0xFFFFFFFF
GENERATIONS = [0, 1, 127, 253, 254, 255, 256, 511, -1]
GEN_CTL_WORD = 4  # int32 index of the control-wave generation in the workspace's control block


def inputs():
    return synth.make("ln_stress_16x64x256x256", device="cuda", shape=SHAPE, normalized_ndim=1, seed=23)


def main(path):
    d = inputs()
    _, ws = nf.alloc_workspace(nf.ln_forward_workspace_size(*SHAPE), "cuda")
    nf.ln_forward_workspace_init(ws)
    out = {}
    for g in GENERATIONS:
        nf.ln_forward(d["x"], d["weight"], d["bias"], variant=0, workspace=ws)  # plants (n, mean, M2) words
        ws.view(torch.int32)[GEN_CTL_WORD:GEN_CTL_WORD + 1].fill_(g)
        y = nf.ln_forward(d["x"], d["weight"], d["bias"], variant=1, workspace=ws)
        torch.cuda.synchronize()
        out[f"y_{g}"] = y.cpu().numpy()
        print(f"generation {g}: done", flush=True)
    out["recomputed"] = np.array(ws[:16].view(torch.int32).cpu().numpy()[3])
    np.savez(path, **out)
    print(f"planted child: ok (recomputed {int(out['recomputed'])})", flush=True)


if __name__ == "__main__":
    main(sys.argv[1])
