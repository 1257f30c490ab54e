"""Seeded synthetic workloads for joint text+image attention.

This module only says what the inputs look like: tensor shapes, the value
distribution, which tokens are outliers, and the integer (row, col) grid
position of every token.  It holds none of the attention, RoPE or
quantization arithmetic, so both the fp64 oracle and the HIP path can take
their inputs from here without sharing any of the method.

Token order of the joint sequence is [text | target image | reference image]:
the pages list the text stream, the noisy image being generated and the
optional reference images, processed separately and then merged by joint
attention ("Speed Up Image Generation with FLUX 3 Image Klein on NVIDIA
Blackwell GPUs", section "FLUX 3 inference with TensorRT LLM VisualGen"); the
order follows that listing.  The pages give no shapes; the sizes
below are the 1024x1024 / 2048x2048 DiT step shapes (16 pixels per latent
token, 512 text tokens, 24 heads of 128) the build is measured on.
"""
from __future__ import annotations

import dataclasses

import numpy as np
import torch

__all__ = ["Workload", "WORKLOADS", "positions", "make_qkv", "outlier_tokens",
           "make_block_mask", "SPARSE_DENSITY", "make_norm_weights"]


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape and value recipe of one joint-attention call."""

    name: str
    batch: int
    heads: int
    head_dim: int
    n_text: int          # text tokens, placed first, all at grid position (0, 0)
    grid: int            # target image is grid x grid latent tokens, row-major
    n_ref: int = 0       # reference-image grids appended after the target
    outlier_frac: float = 0.0   # fraction of tokens whose Q/K/V are scaled
    outlier_scale: float = 8.0
    theta: float = 10000.0

    @property
    def seq_len(self) -> int:
        return self.n_text + self.grid * self.grid * (1 + self.n_ref)

    @property
    def shape(self) -> tuple:
        return (self.batch, self.seq_len, self.heads, self.head_dim)

    def flops(self) -> float:
        """Dense forward flops, QK^T plus PV: 4 * B * H * S^2 * D."""
        s = self.seq_len
        return 4.0 * self.batch * self.heads * s * s * self.head_dim

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    # 16 text + 8x8 image tokens, no outliers: the oracle runs it in milliseconds.
    "tiny": Workload("tiny", 1, 2, 64, 16, 8),
    # 1024x1024 T2I step: 512 text + 64x64 latent grid.
    "t2i_1024": Workload("t2i_1024", 1, 24, 128, 512, 64, outlier_frac=0.01),
    # 2048x2048 T2I step: 512 text + 128x128 latent grid (the measured shape).
    "t2i_2048": Workload("t2i_2048", 1, 24, 128, 512, 128, outlier_frac=0.01),
    # 2048x2048 I2I with guidance: cond/uncond as batch 2, one reference grid.
    "i2i_2048": Workload("i2i_2048", 2, 24, 128, 512, 128, n_ref=1, outlier_frac=0.01),
    # Outlier-free controls of the two T2I shapes.
    "t2i_1024_clean": Workload("t2i_1024_clean", 1, 24, 128, 512, 64),
    "t2i_2048_clean": Workload("t2i_2048_clean", 1, 24, 128, 512, 128),
}


def positions(w: Workload) -> np.ndarray:
    """Integer (row, col) grid position of every token, int32 [S, 2].

    Text tokens sit at (0, 0).  Target token t of the G x G grid sits at
    (t // G, t % G).  Reference grid r (r >= 1) is shifted diagonally by r*G
    on both axes so it shares no coordinate with the target grid.
    """
    g = w.grid
    pos = np.zeros((w.seq_len, 2), dtype=np.int32)
    rc = np.stack(np.divmod(np.arange(g * g, dtype=np.int32), g), axis=1)
    at = w.n_text
    for r in range(1 + w.n_ref):
        pos[at:at + g * g] = rc + r * g
        at += g * g
    return pos


def outlier_tokens(w: Workload, gen: torch.Generator) -> torch.Tensor:
    """Seeded token indices (shared by Q, K, V, every head and batch row)."""
    n = int(round(w.outlier_frac * w.seq_len))
    if n == 0:
        return torch.zeros(0, dtype=torch.int64)
    return torch.randperm(w.seq_len, generator=gen)[:n].sort().values


def make_qkv(w: Workload, seed: int = 0):
    """Q, K, V as bf16 CPU tensors [B, S, H, D] plus the outlier token indices.

    fp32 N(0, 1) draws in the order Q, K, V from one CPU generator seeded with
    `seed`; then the outlier tokens are drawn and scaled by `outlier_scale` in
    fp32; the result is cast to bf16 (round to nearest even).
    """
    gen = torch.Generator(device="cpu").manual_seed(int(seed))
    out = []
    for _ in range(3):
        out.append(torch.randn(w.shape, generator=gen, dtype=torch.float32))
    idx = outlier_tokens(w, gen)
    for t in out:
        if idx.numel():
            t[:, idx] *= w.outlier_scale
    q, k, v = (t.to(torch.bfloat16) for t in out)
    return q, k, v, idx


# Kept fraction of the (128-query x 64-key) blocks in the block-sparse
# workload.  The pages give sparsity only as a parameter (tau = 1.0) and
# end-to-end speedups; read against attention's ~60 % share of DiT time and
# the 12 or 16 dense steps of 50, those speedups put attention in the sparse
# steps at about 2x the dense rate, i.e. about half of the blocks kept.
SPARSE_DENSITY = 0.5


def make_block_mask(w: Workload, density: float = SPARSE_DENSITY, seed: int = 0,
                    q_block: int = 128, k_block: int = 64) -> torch.Tensor:
    """Seeded block mask uint8 [B, H, ceil(S/q_block), ceil(S/k_block)]: each
    block is kept (1) independently with probability `density`, drawn as
    U[0, 1) < density from a CPU generator seeded with `seed`."""
    gen = torch.Generator(device="cpu").manual_seed(int(seed))
    s = w.seq_len
    shape = (w.batch, w.heads, -(-s // q_block), -(-s // k_block))
    return (torch.rand(shape, generator=gen, dtype=torch.float64) < density).to(torch.uint8)


def make_norm_weights(head_dim: int, seed: int = 0):
    """Seeded stand-ins for the learned query/key RMS-norm weights (no trained
    checkpoint here): fp32 [D] vectors g_q, g_k = 1 + 0.1 * N(0, 1), drawn in
    that order from a CPU generator seeded with `seed`."""
    gen = torch.Generator(device="cpu").manual_seed(int(seed))
    gq = 1.0 + 0.1 * torch.randn(head_dim, generator=gen, dtype=torch.float32)
    gk = 1.0 + 0.1 * torch.randn(head_dim, generator=gen, dtype=torch.float32)
    return gq.numpy(), gk.numpy()
