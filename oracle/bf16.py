"""Rounding of fp64 values to bfloat16 (oracle; test infrastructure only).

bfloat16 has fp32's exponent range and 8 significant bits.  The rounding is
to nearest, ties to even, taken once from the fp64 value.  (A cast through
fp32 would round twice: a value just above a bf16 midpoint can first round
onto the midpoint and then, by the tie rule, away from its nearest bf16.)
"""
from __future__ import annotations

import numpy as np
import torch


def bf16_round(x) -> torch.Tensor:
    """Nearest bfloat16 of each fp64 value (ties to even), returned as fp64.

    Normal values 2^e * 1.fffffff have spacing 2^(e-7); below 2^-126 the
    subnormal spacing is 2^-133.  Values beyond the largest finite bf16 round
    to +-inf.  x / step is exact in fp64 (a power-of-two division), so
    np.round (half to even) rounds the exact value once.
    """
    a = torch.as_tensor(x).to(torch.float64).numpy()
    mag = np.abs(a)
    _, e = np.frexp(mag)                         # mag = f * 2^e, f in [0.5, 1)
    e = np.maximum(e - 1, -126)                  # exponent of the leading bit
    step = np.ldexp(1.0, e - 7)
    r = np.round(mag / step) * step
    bf16_max = (2.0 - 2.0 ** -7) * 2.0 ** 127
    # the rounding boundary to infinity is halfway to the next binade's first step
    r = np.where(mag >= bf16_max + 2.0 ** (127 - 8), np.inf, np.minimum(r, bf16_max))
    r = np.where(np.isnan(a), np.nan, r)
    return torch.from_numpy(np.copysign(r, a))
