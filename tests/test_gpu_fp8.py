"""GPU parity of the FP8 path: the RoPE + e4m3 quantizer is compared bit for
bit with the oracle's quantizer, and the FP8 forward against fp64 attention on
the oracle's dequantized inputs (rel-L2 <= 3e-2)."""
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


def _quant_gpu(q, k, v, pos):
    rope = None
    if pos is not None:
        rope = ja.rope_table_2d(torch.from_numpy(pos).to(DEV), q.shape[-1])
    res = ja.quant_rope_fp8(q.to(DEV), k.to(DEV), v.to(DEV), rope)
    torch.cuda.synchronize()
    return [t.cpu().numpy() for t in res]


def _cases():
    return [synth.WORKLOADS["tiny"],
            synth.WORKLOADS["tiny"].replace(name="tiny128", head_dim=128, outlier_frac=0.05),
            synth.Workload("ragged", 2, 3, 64, n_text=7, grid=9, outlier_frac=0.03),
            synth.WORKLOADS["t2i_1024"]]


@pytest.mark.parametrize("w", _cases(), ids=lambda w: w.name)
def test_quantizer_bit_exact(w):
    q, k, v, _ = synth.make_qkv(w, 0)
    pos = synth.positions(w)
    _say(f"quant {w.name} S={w.seq_len} D={w.head_dim}")
    got = _quant_gpu(q, k, v, pos)
    ref = oracle.quant_rope_fp8(q, k, v, pos)
    for name, g, r in zip(("q8", "k8", "v8", "sq", "sk", "sv"), got, ref):
        if g.dtype == np.float32:
            g, r = g.view(np.uint32), r.view(np.uint32)
        mism = int(np.count_nonzero(g != r))
        assert mism == 0, f"{name}: {mism} of {g.size} differ"


def test_quantizer_zero_vectors_and_no_rope():
    w = synth.Workload("zeros", 1, 2, 128, n_text=70, grid=0)
    q, k, v, _ = synth.make_qkv(w, 5)
    v[:, 10] = 0
    q[:, 3, 1] = 0
    _say("quant zero vectors, no rope")
    got = _quant_gpu(q, k, v, None)
    ref = oracle.quant_rope_fp8(q, k, v, None)
    for g, r in zip(got, ref):
        assert np.array_equal(g.view(np.uint8) if g.dtype == np.uint8 else g.view(np.uint32),
                              r.view(np.uint8) if r.dtype == np.uint8 else r.view(np.uint32))
    assert got[5][0, 0, 10] == 1.0 and np.all(got[2][0, 10] == 0)


def _fwd_fp8_from_oracle_codes(q8, k8, v8, sq, sk, sv, **kw):
    args = [torch.from_numpy(np.ascontiguousarray(x)).to(DEV) for x in (q8, k8, v8, sq, sk, sv)]
    res = ja.fwd_fp8(*args, **kw)
    torch.cuda.synchronize()
    return res


@pytest.mark.parametrize("s,d", [(1, 128), (80, 64), (129, 128), (700, 64)])
def test_fp8_forward_ragged(s, d):
    w = synth.Workload("ragged", 1, 2, d, n_text=s, grid=0, outlier_frac=0.02)
    q, k, v, _ = synth.make_qkv(w, seed=s)
    rng = np.random.default_rng(s)
    pos = rng.integers(0, 200, size=(s, 2)).astype(np.int32)
    codes = oracle.quant_rope_fp8(q, k, v, pos)
    _say(f"fp8 fwd ragged S={s} D={d}")
    out = _fwd_fp8_from_oracle_codes(*codes)
    ref, _ = oracle.fp8_attention(*codes)
    assert not torch.isnan(out).any()
    assert rel_l2(out, ref) <= FP8_REL_L2


def test_fp8_full_path_1024():
    # GPU quantizer -> GPU FP8 forward, against oracle quantizer -> fp64 attention.
    w = synth.WORKLOADS["t2i_1024"]
    q, k, v, _ = synth.make_qkv(w, 0)
    pos = synth.positions(w)
    _say("fp8 full path t2i_1024")
    rope = ja.rope_table_2d(torch.from_numpy(pos).to(DEV), 128)
    q8, k8, v8, sq, sk, sv = ja.quant_rope_fp8(q.to(DEV), k.to(DEV), v.to(DEV), rope)
    out, lse = ja.fwd_fp8(q8, k8, v8, sq, sk, sv, return_lse=True)
    torch.cuda.synchronize()
    codes = oracle.quant_rope_fp8(q, k, v, pos)
    ref, ref_lse = oracle.fp8_attention(*codes)
    err = rel_l2(out, ref)
    _say(f"  rel_l2={err:.3e}")
    assert err <= FP8_REL_L2
    assert float((lse.cpu().double() - ref_lse).abs().max()) <= 5e-2


def test_fp8_2048_sampled():
    w = synth.WORKLOADS["t2i_2048"]
    q, k, v, idx = synth.make_qkv(w, 0)
    pos = synth.positions(w)
    rows = sample_rows(w.seq_len, w.n_text, idx, 256, seed=2)
    _say(f"fp8 t2i_2048 sampled rows={len(rows)}")
    codes = oracle.quant_rope_fp8(q, k, v, pos)
    out = _fwd_fp8_from_oracle_codes(*codes).cpu()[:, rows]
    ref, _ = oracle.fp8_attention(*codes, rows=rows)
    err = rel_l2(out, ref)
    _say(f"  rel_l2={err:.3e}")
    assert err <= FP8_REL_L2
