"""GPU parity of the block-sparse FP8 forward against fp64 block-sparse
attention on the oracle's dequantized codes (calls go through the C ABI via
the Python binding)."""
import numpy as np
import pytest
import torch

import joint_attention_attn_amd as ja
import oracle
import synth
from parity_util import FP8_REL_L2, rel_l2, sample_rows

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _say(msg):
    print(msg, flush=True)


def _codes(w, seed, pos=None):
    q, k, v, idx = synth.make_qkv(w, seed)
    codes = oracle.quant_rope_fp8(q, k, v, pos)
    return codes, idx


def _dev(codes):
    return [torch.from_numpy(np.ascontiguousarray(x)).to(DEV) for x in codes]


def _oracle(codes, mask, rows=None):
    q8, k8, v8, sq, sk, sv = codes
    return oracle.block_sparse_attention(oracle.dequantize(q8, sq), oracle.dequantize(k8, sk),
                                         oracle.dequantize(v8, sv), mask, rows=rows)


def _lse_close(got, ref, tol=5e-2):
    got = got.detach().cpu().to(torch.float64)
    inf_ref = torch.isinf(ref)
    assert torch.equal(torch.isinf(got), inf_ref)
    assert (got[inf_ref] < 0).all()
    if (~inf_ref).any():
        assert float((got[~inf_ref] - ref[~inf_ref]).abs().max()) <= tol


@pytest.mark.parametrize("s,d,density", [(80, 64, 0.5), (1000, 128, 0.5), (1100, 64, 0.3),
                                         (1100, 128, 0.7), (2049, 128, 0.5)])
def test_ragged_parity(s, d, density):
    w = synth.Workload("sparse8", 2, 3, d, n_text=s, grid=0, outlier_frac=0.01)
    codes, _ = _codes(w, s)
    mask = synth.make_block_mask(w, density, seed=s)
    mask[0, 0, 0] = 0                                   # an empty query block
    _say(f"fp8 sparse S={s} D={d} density={density}")
    out, lse = ja.fwd_fp8_block_sparse(*_dev(codes), mask.to(DEV), return_lse=True)
    torch.cuda.synchronize()
    ref, ref_lse = _oracle(codes, mask)
    _say(f"  rel_l2={rel_l2(out, ref):.3e}")
    assert rel_l2(out, ref) <= FP8_REL_L2
    assert not out[0, :128, 0].any()
    _lse_close(lse, ref_lse)


def test_all_kept_equals_dense_bit_exact():
    # an all-ones mask stages every tile in order, as the dense kernel does,
    # so without the split of the last round the bits agree
    w = synth.WORKLOADS["t2i_1024"]
    codes, _ = _codes(w, 4, synth.positions(w))
    dc = _dev(codes)
    mask = torch.ones(ja.block_mask_shape(w.batch, w.seq_len, w.heads), dtype=torch.uint8,
                      device=DEV)
    _say("fp8 sparse all-ones vs dense t2i_1024")
    out, lse = ja.fwd_fp8_block_sparse(*dc, mask, return_lse=True, split=False)
    dense, dense_lse = ja.fwd_fp8(*dc, return_lse=True, split=False)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), dense.view(torch.int16))
    assert torch.equal(lse, dense_lse)


@pytest.mark.parametrize("split", [True, False])
def test_nothing_kept(split):
    w = synth.Workload("sparse8_empty", 1, 4, 128, n_text=3000, grid=0)
    codes, _ = _codes(w, 2)
    mask = torch.zeros(ja.block_mask_shape(1, w.seq_len, 4), dtype=torch.uint8, device=DEV)
    _say(f"fp8 sparse empty mask split={split}")
    out, lse = ja.fwd_fp8_block_sparse(*_dev(codes), mask, return_lse=True, split=split)
    torch.cuda.synchronize()
    assert not out.any()
    assert torch.isinf(lse).all() and (lse < 0).all()


def test_split_matches_unsplit():
    w = synth.WORKLOADS["t2i_1024"]
    codes, _ = _codes(w, 8, synth.positions(w))
    dc = _dev(codes)
    mask = synth.make_block_mask(w, 0.5, seed=9)
    mask[0, 5, 3] = 0
    mask_d = mask.to(DEV)
    _say("fp8 sparse split vs unsplit t2i_1024")
    a, la = ja.fwd_fp8_block_sparse(*dc, mask_d, return_lse=True, split=True)
    b, lb = ja.fwd_fp8_block_sparse(*dc, mask_d, return_lse=True, split=False)
    torch.cuda.synchronize()
    assert rel_l2(a, b) <= 5e-3
    _lse_close(la, lb.cpu().to(torch.float64), tol=2e-2)
    # the prepared variant gives the same bits as the one-call forward
    kv8 = ja.prep_kv_fp8(dc[1], dc[2], dc[4], dc[5])
    c, lc = ja.fwd_fp8_block_sparse_prepared(dc[0], dc[3], kv8, mask_d, return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), c.view(torch.int16)) and torch.equal(la, lc)


@pytest.mark.parametrize("name", ["t2i_1024", "t2i_2048"])
def test_full_size_sampled_rows(name):
    # the bench workload: seeded half-density mask, sampled query rows
    w = synth.WORKLOADS[name]
    pos = synth.positions(w)
    codes, idx = _codes(w, 0, pos)
    mask = synth.make_block_mask(w, synth.SPARSE_DENSITY, seed=0)
    _say(f"fp8 sparse full size {name}")
    out, lse = ja.fwd_fp8_block_sparse(*_dev(codes), mask.to(DEV), return_lse=True)
    torch.cuda.synchronize()
    rows = sample_rows(w.seq_len, w.n_text, idx[:8], 48, seed=1)
    ref, ref_lse = _oracle(codes, mask, rows=rows)
    got = out.cpu()[:, torch.as_tensor(rows)]
    _say(f"  rel_l2={rel_l2(got, ref):.3e}")
    assert rel_l2(got, ref) <= FP8_REL_L2
    _lse_close(lse.cpu()[:, :, torch.as_tensor(rows)], ref_lse)
