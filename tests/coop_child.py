"""Run in a child process by test_gpu_coop.py: one ln_forward variant-2 call (a cooperative launch) and one
variant-1 call; prints each call's status and message."""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import torch  # noqa: E402

import normalization_ln_forward_amd as nf  # noqa: E402
from normalization_ln_forward_amd import synth  # noqa: E402

d = synth.make("ln_16x64x256x256", device="cuda", shape=(4, 1 << 18), normalized_ndim=1, seed=9)
for variant in (2, 1):
    try:
        nf.ln_forward(d["x"], d["weight"], d["bias"], variant=variant)
        torch.cuda.synchronize()
        print(f"variant {variant}: status 0", flush=True)
    except nf.NormFwdError as e:
        print(f"variant {variant}: status {e.status}: {e}", flush=True)
