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


def rope_table_fp32(pos, head_dim: int, theta: float = 10000.0) -> np.ndarray:
    """(cos, sin) of every pair angle, computed in fp64 and rounded once to
    fp32: float32 [S, D/2, 2]."""
    ang = rope_angles(pos, head_dim, theta)
    return np.stack([np.cos(ang), np.sin(ang)], axis=-1).astype(np.float32)


def fma32(a, b, c) -> np.ndarray:
    """Correctly rounded fp32 fused multiply-add a*b + c of fp32 arrays.

    The product of two fp32 values is exact in fp64; the fp64 sum s = p + c
    is rounded once, and TwoSum recovers its exact error e (p + c = s + e).
    Rounding s to fp32 can only differ from rounding p + c when s lies
    exactly halfway between two fp32 values and e != 0; then the exact value
    is on e's side of the midpoint.
    """
    a = np.asarray(a, np.float32)
    b = np.asarray(b, np.float32)
    c = np.asarray(c, np.float32)
    p = a.astype(np.float64) * b.astype(np.float64)
    c64 = c.astype(np.float64)
    s = p + c64
    bb = s - p
    e = (p - (s - bb)) + (c64 - bb)
    r = s.astype(np.float32)
    r64 = r.astype(np.float64)
    toward_s = np.nextafter(r, np.where(s > r64, np.float32(np.inf), np.float32(-np.inf)))
    tie = (r64 != s) & ((r64 + toward_s.astype(np.float64)) * 0.5 == s) & (e != 0)
    # at a tie the exact value is above s when e > 0: pick the neighbour above
    above = np.where(r64 > s, r, toward_s)
    below = np.where(r64 > s, toward_s, r)
    return np.where(tie, np.where(e > 0, above, below), r).astype(np.float32)


def rotate_fp32(x, table) -> np.ndarray:
    """RoPE of fp32 x [B, S, H, D] with an fp32 (cos, sin) table [S, D/2, 2],
    in the operation order both kernels use, so that every rounding decision
    taken on the result (bf16 operands, e4m3 codes) is reproducible:
        x' = fma(x, cos, -fl(y sin)),   y' = fma(x, sin, fl(y cos)).
    """
    x = np.asarray(x, np.float32)
    c = table[None, :, None, :, 0]
    s = table[None, :, None, :, 1]
    xe = x[..., 0::2]
    xo = x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = fma32(xe, c, -(xo * s))
    out[..., 1::2] = fma32(xe, s, xo * c)
    return out
