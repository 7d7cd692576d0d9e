"""torch.nn.Module front ends with the pages' constructor arguments.

Each page replaces a model's forward with a custom kernel while keeping the
model's constructor: LayerNorm(normalized_shape) on the LN page, fc +
GroupNorm(num_groups, eps) + LeakyReLU(negative_slope) + x + x on the GN page,
RMSNorm(num_features, eps) on the RMS page.  These classes own the parameters
(initialized as torch initializes the corresponding layers) and call the HIP
library through the binding; they hold no arithmetic of their own and no
fallback path.  Forward only (the library has no backward).
"""
import math

import torch

from . import _lib


class LayerNorm(torch.nn.Module):
    """LayerNorm over the trailing ``normalized_shape`` dims (LN page, turn 1)."""

    def __init__(self, normalized_shape, eps=1e-5, elementwise_affine=True, variant=3, device=None):
        super().__init__()
        if isinstance(normalized_shape, int):
            normalized_shape = (normalized_shape,)
        self.normalized_shape = tuple(int(s) for s in normalized_shape)
        self.eps = float(eps)
        self.variant = int(variant)
        if elementwise_affine:
            self.weight = torch.nn.Parameter(torch.ones(self.normalized_shape, device=device))
            self.bias = torch.nn.Parameter(torch.zeros(self.normalized_shape, device=device))
        else:
            self.register_parameter("weight", None)
            self.register_parameter("bias", None)

    def forward(self, x):
        if tuple(x.shape[x.dim() - len(self.normalized_shape):]) != self.normalized_shape:
            raise ValueError(f"trailing dims of x {tuple(x.shape)} are not {self.normalized_shape}")
        w = None if self.weight is None else self.weight.detach()
        b = None if self.bias is None else self.bias.detach()
        return _lib.ln_forward(x, w, b, eps=self.eps, normalized_ndim=len(self.normalized_shape),
                               variant=self.variant)


class GroupNormLeakyReLUx2(torch.nn.Module):
    """GroupNorm(num_groups) on [N, C] -> LeakyReLU(negative_slope) -> x + x (GN page, turn 1)."""

    def __init__(self, num_channels, num_groups, eps=1e-5, negative_slope=0.01, affine=True, device=None):
        super().__init__()
        if num_channels % num_groups != 0:
            raise ValueError("num_channels must be a multiple of num_groups")
        self.num_groups, self.eps, self.negative_slope = int(num_groups), float(eps), float(negative_slope)
        if affine:
            self.weight = torch.nn.Parameter(torch.ones(num_channels, device=device))
            self.bias = torch.nn.Parameter(torch.zeros(num_channels, device=device))
        else:
            self.register_parameter("weight", None)
            self.register_parameter("bias", None)

    def forward(self, x):
        w = None if self.weight is None else self.weight.detach()
        b = None if self.bias is None else self.bias.detach()
        return _lib.gn_lrelu_x2_forward(x, w, b, self.num_groups, eps=self.eps,
                                        negative_slope=self.negative_slope)


class FcGroupNormLeakyReLUx2(torch.nn.Module):
    """fc(input_size -> hidden_size) -> GroupNorm -> LeakyReLU -> x + x (GN page, turn 1).

    The fc parameters are initialized as torch.nn.Linear initializes them
    (weight and bias uniform in +-1/sqrt(input_size)); the GroupNorm affine
    starts at weight 1, bias 0."""

    def __init__(self, input_size, hidden_size, num_groups, eps=1e-5, negative_slope=0.01, device=None):
        super().__init__()
        if hidden_size % num_groups != 0:
            raise ValueError("hidden_size must be a multiple of num_groups")
        bound = 1.0 / math.sqrt(input_size)
        self.fc_weight = torch.nn.Parameter(torch.empty(hidden_size, input_size, device=device).uniform_(-bound, bound))
        self.fc_bias = torch.nn.Parameter(torch.empty(hidden_size, device=device).uniform_(-bound, bound))
        self.gn_weight = torch.nn.Parameter(torch.ones(hidden_size, device=device))
        self.gn_bias = torch.nn.Parameter(torch.zeros(hidden_size, device=device))
        self.num_groups, self.eps, self.negative_slope = int(num_groups), float(eps), float(negative_slope)

    def forward(self, x):
        return _lib.fc_gn_forward(x, self.fc_weight.detach(), self.fc_bias.detach(), self.gn_weight.detach(),
                                  self.gn_bias.detach(), self.num_groups, eps=self.eps,
                                  negative_slope=self.negative_slope)


class RMSNormChannel(torch.nn.Module):
    """x / sqrt(mean over dim 1 of x^2 + eps), no affine (RMS page, turns 1-2)."""

    def __init__(self, num_features, eps=1e-5):
        super().__init__()
        self.num_features, self.eps = int(num_features), float(eps)

    def forward(self, x):
        if x.dim() < 2 or x.shape[1] != self.num_features:
            raise ValueError(f"x must be [B, {self.num_features}, ...]")
        return _lib.rmsnorm_ch_forward(x, eps=self.eps)
