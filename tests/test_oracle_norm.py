"""Pins of the QK RMS normalization oracle (`oracle.norm`): closed forms,
torch's rms_norm (a library routine), invariances, and the attention with
normalized Q/K."""
import numpy as np
import torch

import oracle
import synth


def test_closed_forms():
    d = 128
    g = np.ones(d)
    for c in (1.0, -4.0, 0.25):
        y = oracle.rms_norm(np.full((1, d), c), g, eps=0.0)
        assert np.array_equal(y, np.full((1, d), np.sign(c)))
    # weights multiply elementwise; eps enters as 1/sqrt(1 + eps) on unit vectors
    gw = np.linspace(0.5, 2.0, d)
    y = oracle.rms_norm(np.ones((1, d)), gw, eps=1e-6)
    np.testing.assert_allclose(y[0], gw / np.sqrt(1 + 1e-6), rtol=1e-15)
    # a one-hot vector e_j becomes sqrt(D) g_j e_j (mean of squares 1/D)
    e = np.zeros((1, d))
    e[0, 5] = 3.0
    y = oracle.rms_norm(e, gw, eps=0.0)
    np.testing.assert_allclose(y[0, 5], np.sqrt(d) * gw[5], rtol=1e-15)
    assert np.count_nonzero(y) == 1


def test_matches_torch_rms_norm():
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((4, 7, 3, 128)) * 3).astype(np.float32)
    g = (1 + 0.1 * rng.standard_normal(128)).astype(np.float32)
    ref = oracle.rms_norm(x, g, 1e-6)
    tref = torch.nn.functional.rms_norm(torch.from_numpy(x).double(), (128,),
                                        torch.from_numpy(g).double(), eps=1e-6).numpy()
    np.testing.assert_allclose(ref, tref, rtol=1e-13, atol=0)


def test_power_of_two_scale_invariance():
    # without eps, scaling x by 2^k changes every intermediate by an exact
    # power of two, so the fp64 result is bit-identical
    rng = np.random.default_rng(5)
    x = rng.standard_normal((5, 64))
    g = rng.uniform(0.5, 1.5, 64)
    y = oracle.rms_norm(x, g, eps=0.0)
    for k in (-8, -1, 3, 10):
        assert np.array_equal(oracle.rms_norm(x * 2.0 ** k, g, eps=0.0), y)


def test_prologue_is_norm_then_rotation_and_keeps_rms():
    w = synth.Workload("normp", 1, 2, 128, n_text=8, grid=4)
    q, _, _, _ = synth.make_qkv(w, 1)
    pos = synth.positions(w)
    g = np.ones(128)
    y = oracle.prologue(q, pos, 10000.0, g, 0.0).numpy()
    np.testing.assert_allclose((y ** 2).mean(axis=-1), 1.0, rtol=1e-13)   # rotation keeps the RMS
    # the order: normalizing after the rotation gives the same (the rotation
    # preserves the sum of squares), rotating a non-normalized vector does not
    y2 = oracle.rms_norm(oracle.apply_rope(q, pos).numpy(), g, 0.0)
    np.testing.assert_allclose(y, y2, rtol=0, atol=1e-13)
    assert not np.allclose(oracle.prologue(q, pos).numpy(), y, atol=1e-3)


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
    qn = oracle.bf16_round(oracle.apply_rope(oracle.rms_norm(q.double().numpy(), gq, 0.0), pos))
    kn = oracle.bf16_round(oracle.apply_rope(oracle.rms_norm(k.double().numpy(), gk, 0.0), pos))
    o3, _ = oracle.attention(qn, kn, v)
    assert torch.equal(o1, o3)
