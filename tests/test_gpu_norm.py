"""GPU parity of the query/key RMS normalization fused into the Q load, the
K/V preparation, the FP8 quantizer and the repair plan: outputs against the
fp64 oracle within tolerance, intermediate products (normalized and rotated
K, codes, the repair set) bit for bit against the oracle's."""
import numpy as np
import pytest
import torch

import joint_attention_attn_amd as ja
import oracle
import synth
from parity_util import (BF16_MAX_ABS, BF16_REL_L2, FP8_REL_L2, max_abs, rel_l2,
                         row_scaled_max_abs, sample_rows)

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
EPS = float(np.float32(1e-6))   # the fp32 epsilon the library receives


def _say(msg):
    print(msg, flush=True)


def _case(s, d, seed, b=2, h=3, outliers=0.01):
    w = synth.Workload("norm", b, h, d, n_text=s, grid=0, outlier_frac=outliers)
    q, k, v, _ = synth.make_qkv(w, seed)
    pos = np.random.default_rng(seed).integers(0, 300, size=(s, 2)).astype(np.int32)
    gq, gk = synth.make_norm_weights(d, seed)
    return q, k, v, pos, gq, gk


def _dev(x):
    return torch.as_tensor(x).to(DEV)


@pytest.mark.parametrize("s,d,strided", [(200, 64, False), (1037, 128, False), (130, 128, True)])
def test_prep_kv_norm_bit_exact(s, d, strided):
    q, k, v, pos, gq, gk = _case(s, d, s)
    if strided:
        kd, vd = (t.permute(0, 2, 1, 3).contiguous().to(DEV).permute(0, 2, 1, 3) for t in (k, v))
    else:
        kd, vd = k.to(DEV), v.to(DEV)
    rope = ja.rope_table_2d(_dev(pos), d)
    _say(f"prep kv with norm S={s} D={d} strided={strided}")
    kv = ja.prep_kv_bf16(kd, vd, rope=rope, k_norm=_dev(gk), norm_eps=EPS).cpu()
    s_pad = (s + 63) // 64 * 64
    kr = kv[: 2 * 2 * 3 * s_pad * d].view(torch.bfloat16).view(2, 3, s_pad, d)
    kref = oracle.rotated_qk(k, pos, norm_g=gk, eps=EPS).to(torch.bfloat16)
    assert torch.equal(kr[:, :, :s].view(torch.int16),
                       kref.permute(0, 2, 1, 3).contiguous().view(torch.int16))
    assert not kr[:, :, s:].view(torch.int16).any()


@pytest.mark.parametrize("s,d", [(300, 64), (1000, 128)])
def test_q_norm_bit_exact(s, d):
    # without RoPE, the forward with q_norm on raw Q equals the forward on the
    # oracle's normalized bf16 Q bit for bit (same Q operands, same K/V)
    q, k, v, pos, gq, gk = _case(s, d, s + 1)
    qn = oracle.rotated_qk(q, None, norm_g=gq, eps=EPS).to(torch.bfloat16)
    kv = ja.prep_kv_bf16(k.to(DEV), v.to(DEV))
    _say(f"q norm bit-exact S={s} D={d}")
    a, la = ja.fwd_bf16_prepared(q.to(DEV), kv, return_lse=True, q_norm=_dev(gq), norm_eps=EPS)
    b, lb = ja.fwd_bf16_prepared(qn.to(DEV), kv, return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert torch.equal(la, lb)


@pytest.mark.parametrize("s,d", [(80, 64), (1037, 128), (4608, 128)])
def test_forward_with_norm_parity(s, d):
    q, k, v, pos, gq, gk = _case(s, d, s + 2, b=1, h=4)
    _say(f"bf16 forward with norm S={s} D={d}")
    out, lse = ja.fwd_bf16(q.to(DEV), k.to(DEV), v.to(DEV), pos, return_lse=True,
                           q_norm=_dev(gq), k_norm=_dev(gk), norm_eps=EPS)
    torch.cuda.synchronize()
    rows = None if s <= 1100 else np.random.default_rng(0).choice(s, 200, replace=False)
    ref, ref_lse = oracle.joint_attention(q, k, v, pos, norm=(gq, gk, EPS), rows=rows)
    got = out.cpu() if rows is None else out.cpu()[:, torch.as_tensor(rows)]
    got_lse = lse.cpu() if rows is None else lse.cpu()[:, :, torch.as_tensor(rows)]
    assert rel_l2(got, ref) <= BF16_REL_L2
    assert row_scaled_max_abs(got, ref) <= BF16_MAX_ABS
    assert max_abs(got_lse, ref_lse) <= 1e-2


@pytest.mark.parametrize("s,d", [(200, 64), (1037, 128)])
def test_quant_with_norm_bit_exact(s, d):
    q, k, v, pos, gq, gk = _case(s, d, s + 3)
    rope = ja.rope_table_2d(_dev(pos), d)
    _say(f"fp8 quantize with norm S={s} D={d}")
    got = ja.quant_rope_fp8(q.to(DEV), k.to(DEV), v.to(DEV), rope=rope, q_norm=_dev(gq),
                            k_norm=_dev(gk), norm_eps=EPS)
    ref = oracle.quant_rope_fp8(q, k, v, pos, norm=(gq, gk, EPS))
    for name, g, r in zip(("q8", "k8", "v8", "sq", "sk", "sv"), got, ref):
        g, r = g.cpu().numpy(), np.asarray(r)
        if g.dtype == np.float32:
            g, r = g.view(np.uint32), r.astype(np.float32).view(np.uint32)
        assert np.array_equal(g, r), name
    # and the FP8 forward on them stays within the FP8 bound of fp64
    # attention on the oracle's codes
    out = ja.fwd_fp8(*got)
    torch.cuda.synchronize()
    ref_o, _ = oracle.fp8_attention(*ref)
    assert rel_l2(out, ref_o) <= FP8_REL_L2


def test_repair_plan_with_norm_bit_exact():
    s, d = 1000, 128
    q, k, v, pos, gq, gk = _case(s, d, 9, b=1, h=2)
    rope = ja.rope_table_2d(_dev(pos), d)
    kd, vd = k.to(DEV), v.to(DEV)
    codes = ja.quant_rope_fp8(q.to(DEV), kd, vd, rope=rope, q_norm=_dev(gq), k_norm=_dev(gk),
                              norm_eps=EPS)
    n = ja.repair_count(0.01, s)
    _say("repair plan with norm")
    rp = ja.fp8_repair_plan(kd, vd, codes[1], codes[2], codes[4], codes[5], n, rope=rope,
                            k_norm=_dev(gk), norm_eps=EPS)
    torch.cuda.synchronize()
    _, k8, v8, _, sk, sv = oracle.quant_rope_fp8(q, k, v, pos, norm=(gq, gk, EPS))
    err = oracle.repair_errors(k, v, pos, k8, v8, sk, sv, norm=(gq, gk, EPS))
    idx = oracle.repair_select(err, n)
    assert np.array_equal(rp.idx.cpu().numpy(), idx)
    kr, vr = oracle.repair_values(k, v, pos, idx, norm=(gq, gk, EPS))
    assert torch.equal(rp.kr.cpu()[:, :, :n].to(torch.float64), kr)
    assert torch.equal(rp.vr.cpu()[:, :, :n].to(torch.float64), vr)


def test_forward_with_norm_2048_sampled():
    # the bench's norm leg: t2i_2048 with seeded norm weights, sampled rows
    # (random, 16 outlier rows, first/last text and last rows) by the oracle
    w = synth.WORKLOADS["t2i_2048"]
    q, k, v, idx = synth.make_qkv(w, 0)
    pos = synth.positions(w)
    gq, gk = synth.make_norm_weights(w.head_dim, 0)
    rope = ja.rope_table_2d(_dev(pos), w.head_dim)
    _say("bf16 forward with norm, t2i_2048")
    out, lse = ja.fwd_bf16(q.to(DEV), k.to(DEV), v.to(DEV), rope=rope, return_lse=True,
                           q_norm=_dev(gq), k_norm=_dev(gk), norm_eps=EPS)
    torch.cuda.synchronize()
    rows = sample_rows(w.seq_len, w.n_text, idx[:16], 64, seed=3)
    ref, ref_lse = oracle.joint_attention(q, k, v, pos, norm=(gq, gk, EPS), rows=rows)
    got = out.cpu()[:, torch.as_tensor(rows)]
    got_lse = lse.cpu()[:, :, torch.as_tensor(rows)]
    _say(f"  rel_l2={rel_l2(got, ref):.3e}")
    assert rel_l2(got, ref) <= BF16_REL_L2
    assert row_scaled_max_abs(got, ref) <= BF16_MAX_ABS
    assert max_abs(got_lse, ref_lse) <= 1e-2
