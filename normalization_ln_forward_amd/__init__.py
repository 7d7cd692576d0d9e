"""normfwd: forward passes of LayerNorm, GroupNorm+LeakyReLU+x2 and channel
RMSNorm (plus fc -> GroupNorm) as hand-written HIP kernels for MI355X
(gfx950), behind the C ABI declared in include/normfwd.h.

The Python functions here are a thin ctypes binding with the same names as
the C entry points; they check arguments, allocate outputs with torch and
enqueue the HIP kernels on the current stream.  ``modules`` holds
torch.nn.Module front ends with the constructor arguments of the layers
the kernels replace.
"""
from ._lib import (  # noqa: F401
    NormFwdError,
    alloc_workspace,
    copy_reference,
    fc_gn_forward,
    gn_lrelu_x2_forward,
    lib,
    ln_forward,
    ln_forward_apply,
    ln_forward_noalloc,
    ln_forward_stats,
    ln_forward_workspace_check,
    ln_forward_workspace_init,
    ln_forward_workspace_size,
    prepare,
    release_cached_workspaces,
    rmsnorm_ch_forward,
    time_next_kernel,
)
from . import modules  # noqa: F401,E402
