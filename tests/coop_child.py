"""Run in a child process by test_gpu_coop.py: an in-place ln_forward variant-2 call (a cooperative launch),
a variant-2 call that is not in place (an ordinary launch) and a variant-1 call; prints each call's status
and message."""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import torch  # noqa: E402

import normalization_ln_forward_amd as nf  # noqa: E402
from normalization_ln_forward_amd import synth  # noqa: E402

d = synth.make("ln_16x64x256x256", device="cuda", shape=(4, 1 << 18), normalized_ndim=1, seed=9)
for name, variant, in_place in (("variant 2 in place", 2, True), ("variant 2", 2, False), ("variant 1", 1, False)):
    x = d["x"].clone()
    try:
        nf.ln_forward(x, d["weight"], d["bias"], variant=variant, out=x if in_place else None)
        torch.cuda.synchronize()
        print(f"{name}: status 0", flush=True)
    except nf.NormFwdError as e:
        print(f"{name}: status {e.status}: {e}", flush=True)
