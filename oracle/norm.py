"""RMS normalization of Q and K over the head dimension (oracle; test
infrastructure only).

The pages fuse "query/key normalization" with RoPE into the epilogue of the
QKV projection ("Speed Up Image Generation with FLUX 3 Image Klein on NVIDIA
Blackwell GPUs", section "GEMM kernel optimization") and give no formula.
Reading taken here: RMSNorm of every (batch, token, head) vector x of length D,
with one learned fp32 weight vector g of length D for Q and one for K (shared
by the heads) and eps = 1e-6:

    y_d = x_d / sqrt(mean(x^2) + eps) * g_d,

applied before RoPE, the normalized value going into the rotation without a
rounding of its own (the epilogue works in fp32).  The result decides a bf16
value or an e4m3 code, so the fp32 evaluation follows one fixed order, the
one the kernels use:

* sum of squares: the D elements form D/8 chunks of 8; chunk c accumulates
  s_c = fma(x, x, s_c) over its elements in order, from 0; the chunk sums are
  then combined pairwise, level by level, partner c ^ k for
  k = 2, 4, ..., D/16, then k = 1 (every level adds the two values of the
  previous level: a butterfly, so every chunk ends with the same total);
* ms = ss / D (exact, D a power of two); r = 1 / sqrt(ms + eps) with IEEE
  fp32 addition, square root and division;
* y_d = fl(fl(x_d * r) * g_d).
"""
from __future__ import annotations

import numpy as np
import torch

from .rope import fma32, rope_table_fp32, rotate_fp32

NORM_EPS = 1e-6


def _levels(chunks: int):
    """Partner offsets of the chunk-sum butterfly, in order."""
    ks = []
    k = 2
    while k < chunks:
        ks.append(k)
        k *= 2
    if chunks > 1:
        ks.append(1)
    return ks


def sum_squares_fp32(x) -> np.ndarray:
    """fp32 sum of squares over the last axis of fp32 x [..., D] in the order
    stated above; returns float32 [...]."""
    x = np.asarray(x, np.float32)
    d = x.shape[-1]
    if d % 8:
        raise ValueError("head_dim must be a multiple of 8")
    ch = d // 8
    xc = x.reshape(x.shape[:-1] + (ch, 8))
    s = np.zeros(x.shape[:-1] + (ch,), np.float32)
    for e in range(8):
        s = fma32(xc[..., e], xc[..., e], s)
    for k in _levels(ch):
        s = (s + s[..., np.arange(ch) ^ k]).astype(np.float32)
    return s[..., 0]


def rms_norm_fp32(x, g, eps: float = NORM_EPS) -> np.ndarray:
    """RMSNorm of fp32 x [..., D] with weight g [D], in the fp32 order stated
    above; returns float32 [..., D]."""
    x = np.asarray(x, np.float32)
    g = np.asarray(g, np.float32)
    d = x.shape[-1]
    ms = sum_squares_fp32(x) * np.float32(1.0 / d)
    r = np.float32(1.0) / np.sqrt((ms + np.float32(eps)).astype(np.float32))
    r = r.astype(np.float32)
    y = (x * r[..., None]).astype(np.float32)
    return (y * g).astype(np.float32)


def rms_norm(x, g, eps: float = NORM_EPS) -> np.ndarray:
    """The same normalization in fp64 (the plain formula), for comparison."""
    x = np.asarray(x, np.float64)
    g = np.asarray(g, np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * g


def prologue_fp32(x, pos=None, theta: float = 10000.0, g=None, eps: float = NORM_EPS,
                  table=None) -> np.ndarray:
    """The fp32 values the kernels round: RMSNorm with weight g (if given),
    then RoPE at positions pos (if given) in `rotate_fp32` order.
    x: [B, S, H, D] (any float dtype); returns float32."""
    x32 = torch.as_tensor(x).to(torch.float32).numpy()
    if g is not None:
        x32 = rms_norm_fp32(x32, g, eps)
    if pos is not None:
        if table is None:
            table = rope_table_fp32(pos, x32.shape[-1], theta)
        x32 = rotate_fp32(x32, table)
    return x32
