"""Pins of the fp64 attention oracle (CPU only): closed forms, invariances,
a library routine (torch's scaled_dot_product_attention in fp64) and a
pure-Python brute force."""
import math
import os

import numpy as np
import pytest
import torch

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(shape, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(shape, generator=g, dtype=torch.float64) * scale


def test_single_key_returns_its_value():
    q, k, v = _rand((2, 1, 3, 64), 0), _rand((2, 1, 3, 64), 1), _rand((2, 1, 3, 64), 2)
    o, lse = oracle.attention(q, k, v)
    assert torch.allclose(o, v, rtol=0, atol=1e-15)
    score = (q * k).sum(-1) / 8.0                     # [B, 1, H]
    assert torch.allclose(lse, score.permute(0, 2, 1), atol=1e-13)


def test_equal_scores_give_mean_of_values():
    s = 37
    q = torch.zeros((1, s, 2, 64), dtype=torch.float64)
    k, v = _rand((1, s, 2, 64), 3), _rand((1, s, 2, 64), 4)
    o, lse = oracle.attention(q, k, v)
    assert torch.allclose(o, v.mean(dim=1, keepdim=True).expand_as(o), atol=1e-14)
    assert torch.allclose(lse, torch.full_like(lse, math.log(s)), atol=1e-14)


def test_rows_sum_to_one():
    q, k = _rand((1, 50, 2, 64), 5, 3.0), _rand((1, 50, 2, 64), 6, 3.0)
    v = torch.ones((1, 50, 2, 64), dtype=torch.float64)
    o, _ = oracle.attention(q, k, v)
    assert torch.allclose(o, v, atol=1e-14)


def test_key_value_permutation_invariance():
    q, k, v = (_rand((1, 45, 2, 64), i) for i in (7, 8, 9))
    perm = torch.randperm(45, generator=torch.Generator().manual_seed(1))
    o1, l1 = oracle.attention(q, k, v)
    o2, l2 = oracle.attention(q, k[:, perm], v[:, perm])
    assert torch.allclose(o1, o2, atol=1e-13) and torch.allclose(l1, l2, atol=1e-13)
    # A mismatched permutation must change the result (guards the test itself).
    o3, _ = oracle.attention(q, k[:, perm], v)
    assert not torch.allclose(o1, o3, atol=1e-3)


def test_token_permutation_equivariance_with_rope():
    w = synth.WORKLOADS["tiny"]
    q, k, v, _ = synth.make_qkv(w, seed=3)
    pos = synth.positions(w)
    perm = torch.randperm(w.seq_len, generator=torch.Generator().manual_seed(2))
    o1, _ = oracle.joint_attention(q, k, v, pos)
    o2, _ = oracle.joint_attention(q[:, perm], k[:, perm], v[:, perm], pos[perm.numpy()])
    assert torch.allclose(o1[:, perm], o2, atol=1e-12)


def test_query_key_rescaling_invariance():
    q, k, v = (_rand((1, 30, 2, 64), i) for i in (10, 11, 12))
    o1, _ = oracle.attention(q, k, v)
    o2, _ = oracle.attention(q * 4.0, k / 4.0, v)
    assert torch.allclose(o1, o2, atol=1e-13)


def test_dominant_key_returns_its_value():
    s, d = 20, 64
    q = torch.zeros((1, s, 1, d), dtype=torch.float64)
    q[..., 0] = 1.0
    k = _rand((1, s, 1, d), 13) * 0.01
    k[0, 11, 0, 0] = 2000.0                           # score 250 above the others
    v = _rand((1, s, 1, d), 14)
    o, _ = oracle.attention(q, k, v)
    assert torch.allclose(o, v[:, 11:12].expand_as(o), atol=1e-12)


def test_two_key_golden_closed_form():
    vals = {}
    for line in open(os.path.join(GOLDEN, "two_key_softmax.txt")):
        if line.strip() and not line.startswith("#"):
            name, *nums = line.split()
            vals[name] = [float(x) for x in nums]
    q = torch.tensor([[vals["q"], vals["q"]]], dtype=torch.float64)[:, :, None, :]
    k = torch.tensor([[vals["k0"], vals["k1"]]], dtype=torch.float64)[:, :, None, :]
    v = torch.tensor([[vals["v0"], vals["v1"]]], dtype=torch.float64)[:, :, None, :]
    o, lse = oracle.attention(q, k, v)
    assert torch.allclose(o[0, 0, 0], torch.tensor(vals["o"], dtype=torch.float64), atol=1e-14)
    assert abs(float(lse[0, 0, 0]) - vals["lse"][0]) < 1e-14


def test_matches_torch_sdpa_fp64_without_rope():
    q, k, v = (_rand((2, 70, 3, 64), i, 2.0) for i in (15, 16, 17))
    o, _ = oracle.joint_attention(q, k, v, pos=None)
    ref = torch.nn.functional.scaled_dot_product_attention(
        q.permute(0, 2, 1, 3), k.permute(0, 2, 1, 3), v.permute(0, 2, 1, 3))
    assert torch.allclose(o, ref.permute(0, 2, 1, 3), atol=1e-13)


def test_zero_positions_make_rope_a_no_op():
    w = synth.WORKLOADS["tiny"]
    q, k, v, _ = synth.make_qkv(w, seed=4)
    zero = np.zeros((w.seq_len, 2), np.int32)
    o1, l1 = oracle.joint_attention(q, k, v, zero)
    o2, l2 = oracle.joint_attention(q, k, v, None)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("seed", [0, 1])
def test_vectorised_matches_brute_force_on_tiny(seed):
    w = synth.WORKLOADS["tiny"].replace(n_text=4, grid=4)   # 20 tokens keeps the loop quick
    q, k, v, _ = synth.make_qkv(w, seed=seed)
    pos = synth.positions(w)
    o, lse = oracle.joint_attention(q, k, v, pos)
    qr = oracle.apply_rope(q, pos).to(torch.bfloat16)
    kr = oracle.apply_rope(k, pos).to(torch.bfloat16)
    ob, lb = oracle.brute_force_attention(qr, kr, v)
    assert torch.allclose(o, ob, rtol=0, atol=1e-12)
    assert torch.allclose(lse, lb, rtol=0, atol=1e-12)


def test_row_subset_is_exact():
    w = synth.WORKLOADS["tiny"]
    q, k, v, _ = synth.make_qkv(w, seed=5)
    pos = synth.positions(w)
    o, lse = oracle.joint_attention(q, k, v, pos)
    rows = np.array([0, 3, 15, 16, 40, 79])
    o2, l2 = oracle.joint_attention(q, k, v, pos, rows=rows)
    assert torch.equal(o[:, rows], o2) and torch.equal(lse[:, :, rows], l2)


def test_rotated_inputs_are_rounded_to_bf16():
    w = synth.WORKLOADS["tiny"]
    q, k, v, _ = synth.make_qkv(w, seed=6)
    pos = synth.positions(w)
    o_r, _ = oracle.joint_attention(q, k, v, pos, round_rotated=True)
    o_p, _ = oracle.joint_attention(q, k, v, pos, round_rotated=False)
    diff = (o_r - o_p).abs().max().item()
    # bf16 rounding of the rotated operands moves the result, but only at the
    # level of bf16's relative precision (2^-8) times the output scale.
    assert 0 < diff < 5e-2


# ---- block-sparse variant ----

def _sparse_case(seed=0, s=300, h=2, d=64):
    w = synth.Workload("sparse", 1, h, d, n_text=s, grid=0, outlier_frac=0.02)
    q, k, v, _ = synth.make_qkv(w, seed)
    rng = np.random.default_rng(seed)
    pos = rng.integers(0, 50, size=(s, 2)).astype(np.int32)
    nq = -(-s // oracle.QUERY_BLOCK)
    nk = -(-s // oracle.KEY_BLOCK)
    return q, k, v, pos, nq, nk


def test_block_sparse_all_ones_is_dense():
    q, k, v, pos, nq, nk = _sparse_case()
    mask = np.ones((1, 2, nq, nk), np.uint8)
    o, l = oracle.block_sparse_attention(q, k, v, mask, pos)
    od, ld = oracle.joint_attention(q, k, v, pos)
    assert torch.allclose(o, od, rtol=0, atol=1e-12) and torch.allclose(l, ld, rtol=0, atol=1e-12)


def test_block_sparse_equals_attention_on_the_kept_keys():
    # every query block keeps its own set of key blocks: the result for its
    # rows is dense attention over exactly those keys (sliced out)
    q, k, v, pos, nq, nk = _sparse_case(seed=3)
    rng = np.random.default_rng(5)
    mask = (rng.random((1, 2, nq, nk)) < 0.4).astype(np.uint8)
    mask[..., 0] = 1                                  # no empty row
    o, l = oracle.block_sparse_attention(q, k, v, mask, pos)
    s = q.shape[1]
    qr = oracle.bf16_round(oracle.apply_rope(q, pos))
    kr = oracle.bf16_round(oracle.apply_rope(k, pos))
    for h in range(2):
        for qb in range(nq):
            r0, r1 = qb * oracle.QUERY_BLOCK, min(s, (qb + 1) * oracle.QUERY_BLOCK)
            keys = np.concatenate([np.arange(kb * oracle.KEY_BLOCK, min(s, (kb + 1) * oracle.KEY_BLOCK))
                                   for kb in range(nk) if mask[0, h, qb, kb]])
            sel = torch.as_tensor(keys, dtype=torch.int64)
            od, ld = oracle.attention(qr[:, r0:r1, h:h + 1], kr[:, sel, h:h + 1], v[:, sel, h:h + 1])
            assert torch.allclose(o[:, r0:r1, h:h + 1], od, rtol=0, atol=1e-12)
            assert torch.allclose(l[:, h:h + 1, r0:r1], ld, rtol=0, atol=1e-12)


def test_block_sparse_empty_row_and_brute_force():
    w = synth.Workload("sparse_tiny", 1, 1, 16, n_text=200, grid=0)
    q, k, v, _ = synth.make_qkv(w, 9)
    mask = np.array([[[[1, 0, 1, 0], [0, 0, 0, 0]]]], np.uint8)   # 2 x 4 blocks of 128 x 64
    o, l = oracle.block_sparse_attention(q, k, v, mask)
    assert torch.equal(o[:, 128:], torch.zeros_like(o[:, 128:]))
    assert torch.isinf(l[:, :, 128:]).all() and (l[:, :, 128:] < 0).all()
    keys = torch.as_tensor(np.r_[0:64, 128:192], dtype=torch.int64)
    ob, lb = oracle.brute_force_attention(q[:, :128:9], k[:, keys], v[:, keys])
    assert torch.allclose(o[:, :128:9], ob, rtol=0, atol=1e-12)
    assert torch.allclose(l[:, :, :128:9], lb, rtol=0, atol=1e-12)
