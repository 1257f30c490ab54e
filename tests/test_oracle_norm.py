"""Pins of the QK RMS normalization oracle (`oracle.norm`): closed forms, the
plain fp64 formula and torch's rms_norm, exact rational arithmetic for the
fp32 evaluation order, invariances, and the attention with normalized Q/K."""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synth


def _round_f32(fr: Fraction) -> np.float32:
    """Correctly rounded (to nearest even) fp32 of an exact rational (normal range)."""
    if fr == 0:
        return np.float32(0.0)
    sign = -1 if fr < 0 else 1
    a = abs(fr)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    scaled = a / Fraction(2) ** (e - 23)            # in [2^23, 2^24)
    m = scaled.numerator // scaled.denominator
    rem = scaled - m
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and m % 2 == 1):
        m += 1
    return np.float32(sign * float(Fraction(m) * Fraction(2) ** (e - 23)))


def _exact_sum_squares(x):
    """The documented order with every operation rounded from its exact value."""
    d = len(x)
    ch = d // 8
    s = []
    for c in range(ch):
        acc = np.float32(0.0)
        for e in range(8):
            v = Fraction(float(x[8 * c + e]))
            acc = _round_f32(v * v + Fraction(float(acc)))
        s.append(acc)
    ks = []
    k = 2
    while k < ch:
        ks.append(k)
        k *= 2
    ks.append(1)
    for k in ks:
        s = [_round_f32(Fraction(float(s[c])) + Fraction(float(s[c ^ k]))) for c in range(ch)]
    return s[0]


@pytest.mark.parametrize("d", [64, 128])
def test_sum_squares_order_is_exact(d):
    # values over a wide dynamic range, so that the order of the additions
    # decides rounding; the oracle's fp32 tree equals the exact-rational one
    rng = np.random.default_rng(d)
    x = (rng.standard_normal((6, d)) * np.exp(rng.uniform(-6, 6, (6, d)))).astype(np.float32)
    got = oracle.sum_squares_fp32(x)
    for i in range(6):
        assert got[i] == _exact_sum_squares(x[i]), i
    # and the order matters: a plain sequential fp32 sum differs somewhere
    seq = np.zeros(6, np.float32)
    for j in range(d):
        seq = (seq + x[:, j] * x[:, j]).astype(np.float32)
    assert (seq != got).any()


def test_closed_forms():
    d = 128
    g = np.ones(d, np.float32)
    for c in (1.0, -4.0, 0.25):
        x = np.full((1, d), c, np.float32)
        y = oracle.rms_norm_fp32(x, g, eps=0.0)
        assert np.array_equal(y, np.full((1, d), np.sign(c), np.float32))
    # weights multiply elementwise; eps enters as 1/sqrt(1 + eps) on unit vectors
    gw = np.linspace(0.5, 2.0, d).astype(np.float32)
    y = oracle.rms_norm_fp32(np.ones((1, d), np.float32), gw, eps=1e-6)
    np.testing.assert_allclose(y[0], gw / np.sqrt(1 + 1e-6), rtol=2 ** -22)


def test_matches_fp64_formula_and_torch():
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((4, 7, 3, 128)) * 3).astype(np.float32)
    g = (1 + 0.1 * rng.standard_normal(128)).astype(np.float32)
    ref = oracle.rms_norm(x, g, 1e-6)
    tref = torch.nn.functional.rms_norm(torch.from_numpy(x).double(), (128,),
                                        torch.from_numpy(g).double(), eps=1e-6).numpy()
    np.testing.assert_allclose(ref, tref, rtol=1e-13, atol=0)
    got = oracle.rms_norm_fp32(x, g, 1e-6)
    # a few fp32 roundings (sum, sqrt, division, two products)
    np.testing.assert_allclose(got, ref, rtol=2 ** -20, atol=0)


def test_power_of_two_scale_invariance():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((5, 64)).astype(np.float32)
    g = rng.uniform(0.5, 1.5, 64).astype(np.float32)
    y = oracle.rms_norm_fp32(x, g, eps=0.0)
    for k in (-8, -1, 3, 10):
        assert np.array_equal(oracle.rms_norm_fp32(x * np.float32(2.0 ** k), g, eps=0.0), y)


def test_prologue_is_norm_then_rotation_and_keeps_rms():
    w = synth.Workload("normp", 1, 2, 128, n_text=8, grid=4)
    q, _, _, _ = synth.make_qkv(w, 1)
    pos = synth.positions(w)
    g = np.ones(128, np.float32)
    y = oracle.prologue_fp32(q, pos, 10000.0, g, 0.0)
    ms = (y.astype(np.float64) ** 2).mean(axis=-1)
    np.testing.assert_allclose(ms, 1.0, rtol=1e-5)      # rotation preserves the RMS


def test_attention_with_norm_ignores_the_scale_of_q_and_k():
    w = synth.Workload("norma", 1, 2, 64, n_text=40, grid=4)
    q, k, v, _ = synth.make_qkv(w, 2)
    pos = synth.positions(w)
    rng = np.random.default_rng(7)
    gq = rng.uniform(0.5, 1.5, 64).astype(np.float32)
    gk = rng.uniform(0.5, 1.5, 64).astype(np.float32)
    o1, l1 = oracle.joint_attention(q, k, v, pos, norm=(gq, gk, 0.0))
    o2, l2 = oracle.joint_attention(q * 4, k * 0.5, v, pos, norm=(gq, gk, 0.0))
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    # and equals attention on the normalized, rotated, bf16-rounded Q/K
    qn = torch.from_numpy(oracle.prologue_fp32(q, pos, 10000.0, gq, 0.0)).to(torch.bfloat16)
    kn = torch.from_numpy(oracle.prologue_fp32(k, pos, 10000.0, gk, 0.0)).to(torch.bfloat16)
    o3, _ = oracle.attention(qn, kn, v)
    assert torch.equal(o1, o3)
