"""2D-axial rotary position embedding, fp64 (oracle; test infrastructure only).

The pages say RoPE is fused into the QKV projection epilogue ("Speed Up Image
Generation with FLUX 3 Image Klein on NVIDIA Blackwell GPUs", section "GEMM
kernel optimization") but give no formula.  Reading taken here:

* each head vector of length D is split in two halves; the first half is
  rotated by the token's grid row, the second half by its grid column;
* within a half, adjacent elements (2k, 2k+1), k < D/4, form a pair rotated
  by angle pos * w_k with w_k = theta^(-2k/(D/2)) = theta^(-4k/D), theta=1e4:
  the 1-D rotary embedding of dimension D/2 on each axis;
* a pair (x, y) maps to (x cos a - y sin a, x sin a + y cos a).

Everything here is evaluated in fp64, as the plain formula.
"""
from __future__ import annotations

import numpy as np
import torch


def rope_angles(pos, head_dim: int, theta: float = 10000.0) -> np.ndarray:
    """Rotation angle of every pair, fp64 [S, D/2].

    Pair p < D/4 belongs to the row half (frequency index k = p); pair
    p >= D/4 to the column half (k = p - D/4).
    """
    pos = np.asarray(pos, dtype=np.int64)
    if head_dim % 4:
        raise ValueError("head_dim must be a multiple of 4 for 2D-axial RoPE")
    quarter = head_dim // 4
    k = np.arange(quarter, dtype=np.float64)
    w = np.power(np.float64(theta), -2.0 * k / (head_dim / 2))        # [D/4]
    row = pos[:, 0:1].astype(np.float64) * w[None, :]
    col = pos[:, 1:2].astype(np.float64) * w[None, :]
    return np.concatenate([row, col], axis=1)                          # [S, D/2]


def apply_rope(x, pos, theta: float = 10000.0) -> torch.Tensor:
    """Rotate x [B, S, H, D] (any float dtype) in fp64; returns fp64."""
    x = torch.as_tensor(x).to(torch.float64)
    d = x.shape[-1]
    ang = torch.from_numpy(rope_angles(pos, d, theta))                 # [S, D/2]
    c = torch.cos(ang)[None, :, None, :]
    s = torch.sin(ang)[None, :, None, :]
    xe, xo = x[..., 0::2], x[..., 1::2]
    out = torch.empty_like(x)
    out[..., 0::2] = xe * c - xo * s
    out[..., 1::2] = xe * s + xo * c
    return out
