"""RMS normalization of Q and K over the head dimension, and the Q/K
prologue (oracle; test infrastructure only).

The pages fuse "query/key normalization" with RoPE into the epilogue of the
QKV projection ("Speed Up Image Generation with FLUX 3 Image Klein on NVIDIA
Blackwell GPUs", section "GEMM kernel optimization") and give no formula.
Reading taken here: RMSNorm of every (batch, token, head) vector x of length D,
with one learned weight vector g of length D for Q and one for K (shared by
the heads) and eps = 1e-6:

    y_d = x_d / sqrt(mean(x^2) + eps) * g_d,

applied before RoPE; the normalized value goes into the rotation with no
rounding of its own (the epilogue keeps it in full precision).  Evaluated in
fp64 as the plain formula.
"""
from __future__ import annotations

import numpy as np
import torch

from .rope import apply_rope

NORM_EPS = 1e-6


def rms_norm(x, g, eps: float = NORM_EPS) -> np.ndarray:
    """RMSNorm of x [..., D] with weight g [D], fp64."""
    x = np.asarray(x, np.float64)
    g = np.asarray(g, np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * g


def prologue(x, pos=None, theta: float = 10000.0, g=None, eps: float = NORM_EPS) -> torch.Tensor:
    """What the QKV epilogue does to Q or K before attention, in fp64:
    RMSNorm with weight g (if given), then RoPE at positions pos (if given).
    x: [B, S, H, D] of any float dtype; returns fp64 [B, S, H, D] (unrounded)."""
    y = torch.as_tensor(x).to(torch.float64)
    if g is not None:
        y = torch.from_numpy(rms_norm(y.numpy(), g, eps))
    if pos is not None:
        y = apply_rope(y, pos, theta)
    return y
