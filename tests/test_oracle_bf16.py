"""Pins of the oracle's single rounding from fp64 to bfloat16 (CPU only):
torch's fp32 -> bf16 cast (a library routine, a single rounding on values
that are exact in fp32), exact rational nearest-even rounding, and the
double-rounding case that a cast through fp32 gets wrong."""
from fractions import Fraction

import numpy as np
import torch

import oracle


def _bf16_neighbours(x: float):
    """The two bf16 values around x (exact, via the fp32 bit pattern)."""
    lo = torch.tensor([x], dtype=torch.float64).to(torch.float32)
    bits = lo.view(torch.int32).item() & ~0xFFFF
    a = torch.tensor([bits], dtype=torch.int32).view(torch.float32).double().item()
    step = 2.0 ** (np.frexp(abs(a))[1] - 8) if a != 0 else 2.0 ** -133
    return sorted({a, a + step if x >= 0 else a - step, a - step if x >= 0 else a + step})


def test_matches_torch_cast_on_fp32_values():
    g = torch.Generator().manual_seed(0)
    x = torch.randn(200000, generator=g) * torch.exp(torch.randn(200000, generator=g) * 8)
    x = torch.cat([x, torch.tensor([0.0, -0.0, 1e-39, -3e-40, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8])])
    assert torch.equal(oracle.bf16_round(x.double()), x.to(torch.bfloat16).double())


def test_nearest_even_by_exact_arithmetic():
    rng = np.random.default_rng(1)
    xs = rng.standard_normal(3000) * np.exp(rng.uniform(-20, 20, 3000))
    got = oracle.bf16_round(xs).numpy()
    for x, r in zip(xs, got):
        cands = _bf16_neighbours(float(x))
        ex = Fraction(float(x))
        best = min(cands, key=lambda c: (abs(Fraction(c) - ex),
                                         int(abs(c) / 2.0 ** (np.frexp(abs(c))[1] - 8)) & 1))
        assert r == best, (x, r, best)


def test_single_rounding_where_fp32_would_round_twice():
    # 1 + 2^-8 + 2^-30 lies just above the midpoint of 1 and 1 + 2^-7; through
    # fp32 it first becomes the midpoint, then rounds to even (1.0)
    x = torch.tensor([1 + 2 ** -8 + 2 ** -30, -(1 + 2 ** -8 + 2 ** -30), 1 + 2 ** -8],
                     dtype=torch.float64)
    assert oracle.bf16_round(x).tolist() == [1 + 2 ** -7, -(1 + 2 ** -7), 1.0]
    assert x.to(torch.bfloat16).double()[0].item() == 1.0
