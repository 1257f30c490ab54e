"""Pins of the fp64 2D-axial RoPE oracle (CPU only).

Each test checks the oracle against something other than its own formula:
identities of rotations, closed forms, and GPT-J's interleaved rotary
embedding from `transformers` (a library routine) on each axis half.
"""
import math

import numpy as np
import pytest
import torch

import oracle

D = 64


def _rand(shape, seed=0):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(shape, generator=g, dtype=torch.float64)


def _pos(s, seed=1, hi=300):
    rng = np.random.default_rng(seed)
    return rng.integers(0, hi, size=(s, 2)).astype(np.int32)


def test_zero_position_is_identity():
    x = _rand((2, 7, 3, D))
    out = oracle.apply_rope(x, np.zeros((7, 2), np.int32))
    assert torch.equal(out, x)


def test_pair_norms_preserved():
    x = _rand((1, 9, 2, D))
    out = oracle.apply_rope(x, _pos(9))
    n_in = x[..., 0::2] ** 2 + x[..., 1::2] ** 2
    n_out = out[..., 0::2] ** 2 + out[..., 1::2] ** 2
    assert torch.allclose(n_in, n_out, rtol=1e-14, atol=1e-14)


def test_relative_position_property():
    # <R(p) q, R(p') k> = <q, R(p' - p) k> for every (row, col) pair p, p'.
    q = _rand((1, 1, 1, D), 3)
    k = _rand((1, 1, 1, D), 4)
    for p, pp in [((3, 5), (10, 2)), ((0, 0), (7, 9)), ((120, 64), (5, 127))]:
        lhs = (oracle.apply_rope(q, np.array([p], np.int32)) *
               oracle.apply_rope(k, np.array([pp], np.int32))).sum()
        d = np.array([[pp[0] - p[0], pp[1] - p[1]]], np.int32)
        rhs = (q * oracle.apply_rope(k, d)).sum()
        assert abs(float(lhs - rhs)) < 1e-12 * max(1.0, abs(float(lhs)))


def test_axes_act_on_their_own_half():
    x = _rand((1, 4, 2, D), 5)
    rows_only = np.array([[3, 0], [17, 0], [100, 0], [1, 0]], np.int32)
    out = oracle.apply_rope(x, rows_only)
    assert torch.equal(out[..., D // 2:], x[..., D // 2:])
    assert not torch.allclose(out[..., :D // 2], x[..., :D // 2])
    cols_only = rows_only[:, ::-1].copy()
    out = oracle.apply_rope(x, cols_only)
    assert torch.equal(out[..., :D // 2], x[..., :D // 2])


def test_first_pair_closed_form():
    # Frequency index 0 has w_0 = 1: e_0 at row r becomes (cos r, sin r, 0...),
    # and e_{D/2} at column c becomes (cos c, sin c) at dims D/2, D/2+1.
    for r in [1, 2, 77]:
        e = torch.zeros((1, 1, 1, D), dtype=torch.float64)
        e[..., 0] = 1.0
        out = oracle.apply_rope(e, np.array([[r, 0]], np.int32))[0, 0, 0]
        assert math.isclose(out[0], math.cos(r), abs_tol=1e-15)
        assert math.isclose(out[1], math.sin(r), abs_tol=1e-15)
        assert torch.count_nonzero(out[2:]) == 0
        e = torch.zeros((1, 1, 1, D), dtype=torch.float64)
        e[..., D // 2 + 1] = 1.0          # the odd element of the first column pair
        out = oracle.apply_rope(e, np.array([[0, r]], np.int32))[0, 0, 0]
        assert math.isclose(out[D // 2], -math.sin(r), abs_tol=1e-15)
        assert math.isclose(out[D // 2 + 1], math.cos(r), abs_tol=1e-15)


def test_theta_one_rotates_every_pair_by_position():
    # With theta = 1 every frequency is 1, so every pair of the row half turns
    # by the row and every pair of the column half by the column.
    x = torch.zeros((1, 1, 1, D), dtype=torch.float64)
    x[..., 0::2] = 1.0
    out = oracle.apply_rope(x, np.array([[2, 5]], np.int32), theta=1.0)[0, 0, 0]
    half = D // 2
    assert torch.allclose(out[0:half:2], torch.full((half // 2,), math.cos(2.0), dtype=torch.float64))
    assert torch.allclose(out[1:half:2], torch.full((half // 2,), math.sin(2.0), dtype=torch.float64))
    assert torch.allclose(out[half::2], torch.full((half // 2,), math.cos(5.0), dtype=torch.float64))
    assert torch.allclose(out[half + 1::2], torch.full((half // 2,), math.sin(5.0), dtype=torch.float64))


@pytest.mark.parametrize("head_dim", [64, 128])
def test_matches_gptj_rotary_on_each_axis(head_dim):
    # GPT-J's rotary embedding (transformers) rotates interleaved pairs with
    # inverse frequencies 10000^(-2i/dim).  2D-axial RoPE is that embedding of
    # dim D/2 applied to the row half with row positions and to the column
    # half with column positions.  The library builds its tables in fp32.
    gptj = pytest.importorskip("transformers.models.gptj.modeling_gptj")
    s, h = 40, 3
    x = _rand((1, s, h, head_dim), 7).to(torch.float32)
    pos = _pos(s, 8, hi=256)
    half = head_dim // 2
    table = gptj.create_sinusoidal_positions(256, half)          # [P, half] = [sin | cos]
    expect = torch.empty_like(x)
    for axis in range(2):
        sincos = table[torch.from_numpy(pos[:, axis].astype(np.int64))][None]   # [1, S, half]
        sin, cos = torch.split(sincos, half // 2, dim=-1)
        part = x[..., axis * half:(axis + 1) * half]
        expect[..., axis * half:(axis + 1) * half] = gptj.apply_rotary_pos_emb(part, sin, cos)
    got = oracle.apply_rope(x, pos)
    assert torch.allclose(got, expect.to(torch.float64), rtol=0, atol=2e-4)
