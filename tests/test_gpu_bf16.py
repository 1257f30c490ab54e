"""GPU parity of the RoPE table and the BF16 joint-attention forward against
the fp64 oracle (calls go through the C ABI via the Python binding)."""
import math

import numpy as np
import pytest
import torch

import joint_attention_attn_amd as ja
import oracle
import synth
from parity_util import (BF16_MAX_ABS, BF16_REL_L2, max_abs, rel_l2,
                         row_scaled_max_abs, sample_rows)

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _say(msg):
    print(msg, flush=True)


def _gpu_inputs(w, seed):
    q, k, v, idx = synth.make_qkv(w, seed)
    pos = synth.positions(w)
    return q, k, v, idx, pos


def _run_bf16(q, k, v, pos, theta=10000.0, **kw):
    qd, kd, vd = (t.to(DEV) for t in (q, k, v))
    rope = None
    if pos is not None:
        rope = ja.rope_table_2d(torch.from_numpy(pos).to(DEV), q.shape[-1], theta)
    out = ja.fwd_bf16(qd, kd, vd, rope, **kw)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("name,d", [("tiny", 64), ("t2i_2048", 128), ("i2i_2048", 128)])
def test_rope_table_bit_exact(name, d):
    w = synth.WORKLOADS[name].replace(head_dim=d)
    pos = synth.positions(w)
    _say(f"rope table {name} D={d} S={w.seq_len}")
    got = ja.rope_table_2d(torch.from_numpy(pos).to(DEV), d).cpu().numpy()
    ref = oracle.rope_table_fp32(pos, d)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


def test_tiny_full_parity():
    w = synth.WORKLOADS["tiny"]
    q, k, v, _, pos = _gpu_inputs(w, 0)
    _say("bf16 tiny")
    out, lse = _run_bf16(q, k, v, pos, return_lse=True)
    ref, ref_lse = oracle.joint_attention(q, k, v, pos)
    assert rel_l2(out, ref) <= BF16_REL_L2
    assert max_abs(out, ref) <= BF16_MAX_ABS
    assert max_abs(lse, ref_lse) <= 1e-2


@pytest.mark.parametrize("s,d", [(1, 64), (2, 128), (63, 64), (64, 128), (65, 64),
                                 (127, 128), (129, 128), (200, 64), (1037, 128)])
def test_ragged_lengths(s, d):
    w = synth.Workload("ragged", 2, 3, d, n_text=s, grid=0)
    q, k, v, _ = synth.make_qkv(w, seed=s)
    rng = np.random.default_rng(s)
    pos = rng.integers(0, 200, size=(s, 2)).astype(np.int32)
    _say(f"bf16 ragged S={s} D={d}")
    out, lse = _run_bf16(q, k, v, pos, return_lse=True)
    ref, ref_lse = oracle.joint_attention(q, k, v, pos)
    assert rel_l2(out, ref) <= BF16_REL_L2
    assert max_abs(out, ref) <= BF16_MAX_ABS
    assert max_abs(lse, ref_lse) <= 1e-2


def test_no_rope_and_custom_scale():
    w = synth.Workload("norope", 1, 2, 128, n_text=300, grid=0)
    q, k, v, _ = synth.make_qkv(w, seed=11)
    _say("bf16 no-rope scale=0.05")
    out = _run_bf16(q, k, v, None, softmax_scale=0.05)
    ref, _ = oracle.joint_attention(q, k, v, None, scale=0.05)
    assert rel_l2(out, ref) <= BF16_REL_L2 and max_abs(out, ref) <= BF16_MAX_ABS


def test_strided_bhsd_layout():
    # Q/K/V/O as [B, H, S, D] memory viewed as [B, S, H, D].
    w = synth.Workload("strided", 2, 4, 64, n_text=8, grid=10)
    q, k, v, _ = synth.make_qkv(w, seed=12)
    pos = synth.positions(w)
    qd, kd, vd = (t.permute(0, 2, 1, 3).contiguous().to(DEV).permute(0, 2, 1, 3) for t in (q, k, v))
    out = torch.empty((2, 4, w.seq_len, 64), dtype=torch.bfloat16, device=DEV).permute(0, 2, 1, 3)
    rope = ja.rope_table_2d(torch.from_numpy(pos).to(DEV), 64)
    _say("bf16 strided BHSD")
    ja.fwd_bf16(qd, kd, vd, rope, out=out)
    torch.cuda.synchronize()
    ref, _ = oracle.joint_attention(q, k, v, pos)
    assert rel_l2(out, ref) <= BF16_REL_L2 and max_abs(out, ref) <= BF16_MAX_ABS


def test_closed_forms_on_gpu():
    _say("bf16 closed forms")
    # single key: O = V exactly
    w = synth.Workload("one", 1, 2, 128, n_text=1, grid=0)
    q, k, v, _ = synth.make_qkv(w, seed=13)
    out = _run_bf16(q, k, v, np.array([[5, 7]], np.int32))
    assert torch.equal(out.cpu(), v)
    # Q = 0: O = mean(V); V = 1: O = 1
    w = synth.Workload("mean", 1, 2, 64, n_text=333, grid=0)
    q, k, v, _ = synth.make_qkv(w, seed=14)
    pos = np.zeros((333, 2), np.int32)
    out = _run_bf16(torch.zeros_like(q), k, v, pos)
    mean = v.to(torch.float64).mean(dim=1, keepdim=True).expand(v.shape)
    assert max_abs(out, mean) <= 4e-3
    out = _run_bf16(q, k, torch.ones_like(v), pos)
    assert torch.equal(out.cpu(), torch.ones_like(v))


def test_deterministic_and_fully_written():
    w = synth.WORKLOADS["t2i_1024"].replace(heads=4)
    q, k, v, _, pos = _gpu_inputs(w, 3)
    qd, kd, vd = (t.to(DEV) for t in (q, k, v))
    rope = ja.rope_table_2d(torch.from_numpy(pos).to(DEV), 128)
    _say("bf16 determinism")
    outs = []
    for _ in range(3):
        o = torch.full(q.shape, float("nan"), dtype=torch.bfloat16, device=DEV)
        ja.fwd_bf16(qd, kd, vd, rope, out=o)
        outs.append(o)
    torch.cuda.synchronize()
    assert not torch.isnan(outs[0]).any()
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[1], outs[2])


@pytest.mark.parametrize("name", ["t2i_1024", "t2i_1024_clean"])
def test_1024_full_parity(name):
    w = synth.WORKLOADS[name]
    q, k, v, idx, pos = _gpu_inputs(w, 0)
    _say(f"bf16 {name} full")
    out, lse = _run_bf16(q, k, v, pos, return_lse=True)
    ref, ref_lse = oracle.joint_attention(q, k, v, pos)
    err = rel_l2(out, ref)
    _say(f"  rel_l2={err:.3e} max_abs={max_abs(out, ref):.3e} "
         f"row_scaled={row_scaled_max_abs(out, ref):.3e}")
    assert err <= BF16_REL_L2
    if w.outlier_frac == 0:
        assert max_abs(out, ref) <= BF16_MAX_ABS
    else:
        assert row_scaled_max_abs(out, ref) <= BF16_MAX_ABS
    assert max_abs(lse, ref_lse) <= 2e-2


@pytest.mark.parametrize("name,n_rows", [("t2i_2048", 256), ("t2i_2048_clean", 256),
                                         ("i2i_2048", 96)])
def test_2048_sampled_parity(name, n_rows):
    # Full-size launch (the benchmarked configuration); the oracle evaluates a
    # seeded sample of query rows exactly (rows are independent).
    w = synth.WORKLOADS[name]
    q, k, v, idx, pos = _gpu_inputs(w, 0)
    rows = sample_rows(w.seq_len, w.n_text, idx, n_rows, seed=1)
    _say(f"bf16 {name} sampled rows={len(rows)}")
    out, lse = _run_bf16(q, k, v, pos, return_lse=True)
    out = out.cpu()[:, rows]
    lse = lse.cpu()[:, :, rows]
    ref, ref_lse = oracle.joint_attention(q, k, v, pos, rows=rows)
    err = rel_l2(out, ref)
    _say(f"  rel_l2={err:.3e} max_abs={max_abs(out, ref):.3e} "
         f"row_scaled={row_scaled_max_abs(out, ref):.3e}")
    assert err <= BF16_REL_L2
    if w.outlier_frac == 0:
        assert max_abs(out, ref) <= BF16_MAX_ABS
    else:
        assert row_scaled_max_abs(out, ref) <= BF16_MAX_ABS
    assert max_abs(lse, ref_lse) <= 2e-2


def test_split_last_round_parity():
    # A shape whose last round of workgroups is mostly idle, so the forward
    # splits those work items over key ranges and merges them (the items of
    # the last head's upper query blocks).  Checked against the oracle on
    # rows of split items and of whole items, and against the unsplit launch.
    base = synth.WORKLOADS["t2i_1024"]
    w = ws = None
    for heads in range(8, 65):   # first head count for which a split is planned
        w = base.replace(heads=heads)
        ws = ja.fwd_bf16_workspace_bytes(w.batch, w.seq_len, heads, 128)
        if ws:
            break
    assert ws, "no split planned for any head count"
    q, k, v, idx, pos = _gpu_inputs(w, 5)
    _say(f"bf16 split: S={w.seq_len} H={w.heads} workspace={ws} B")
    out, lse = _run_bf16(q, k, v, pos, return_lse=True)
    out_ns, lse_ns = _run_bf16(q, k, v, pos, return_lse=True, split=False)
    rng = np.random.default_rng(2)
    rows = np.unique(np.concatenate([rng.choice(w.seq_len, 96, replace=False),
                                     np.arange(w.seq_len - 8, w.seq_len)]))
    ref, ref_lse = oracle.joint_attention(q, k, v, pos, rows=rows)
    got, got_lse = out.cpu()[:, rows], lse.cpu()[:, :, rows]
    _say(f"  rel_l2={rel_l2(got, ref):.3e} vs unsplit {rel_l2(out.cpu(), out_ns.cpu()):.3e}")
    assert rel_l2(got, ref) <= BF16_REL_L2
    assert row_scaled_max_abs(got, ref) <= BF16_MAX_ABS
    assert max_abs(got_lse, ref_lse) <= 2e-2
    # The two launches round P to bf16 against different running maxima (each
    # key range of a split item has its own), so they differ by bf16 rounding:
    # about 2^-9 relative in the row sum, a few 1e-3 in the LSE.
    assert rel_l2(out.cpu(), out_ns.cpu()) <= 2e-3
    assert max_abs(lse, lse_ns) <= 1e-2


def _slot_key(p):
    # key of P-operand slot p in a 16-key group (the V^T order the header documents)
    return 4 * (p // 8) + (p % 8 if p % 8 < 4 else p % 8 + 4)


# head counts 3, 6 and 4: workgroups of one, two and four heads
@pytest.mark.parametrize("s,d,strided,h", [(200, 64, False, 3), (1037, 128, False, 3),
                                           (130, 128, True, 3), (300, 128, False, 4),
                                           (130, 64, True, 6)])
def test_prep_kv_bit_exact(s, d, strided, h):
    # rotated K equals the oracle's bf16-rounded rotation bit for bit; V^T is
    # V transposed in the documented key order; padding is zero
    w = synth.Workload("prep", 2, h, d, n_text=s, grid=0)
    q, k, v, _ = synth.make_qkv(w, seed=21)
    pos = np.random.default_rng(s).integers(0, 300, size=(s, 2)).astype(np.int32)
    if strided:
        kd, vd = (t.permute(0, 2, 1, 3).contiguous().to(DEV).permute(0, 2, 1, 3) for t in (k, v))
    else:
        kd, vd = k.to(DEV), v.to(DEV)
    rope = ja.rope_table_2d(torch.from_numpy(pos).to(DEV), d)
    _say(f"prep kv S={s} D={d} H={h} strided={strided}")
    kv = ja.prep_kv_bf16(kd, vd, rope).cpu()
    s_pad = (s + 63) // 64 * 64
    n = 2 * h * s_pad * d
    kr = kv[: 2 * n].view(torch.bfloat16).view(2, h, s_pad, d)
    vt = kv[2 * n:].view(torch.bfloat16).view(2, h, d, s_pad)
    table = oracle.rope_table_fp32(pos, d)
    kref = torch.from_numpy(oracle.rotate_fp32(k.float().numpy(), table)).to(torch.bfloat16)
    assert torch.equal(kr[:, :, :s].view(torch.int16), kref.permute(0, 2, 1, 3).contiguous().view(torch.int16))
    assert not kr[:, :, s:].view(torch.int16).any()
    order = torch.tensor([16 * (j // 16) + _slot_key(j % 16) for j in range(s_pad)])
    vpad = torch.zeros((2, s_pad, h, d), dtype=torch.bfloat16)
    vpad[:, :s] = v
    vref = vpad[:, order].permute(0, 2, 3, 1)            # [B, H, D, S_pad]
    assert torch.equal(vt.view(torch.int16), vref.contiguous().view(torch.int16))


def test_tensors_past_32_bit_element_offsets():
    # Q, K, V and O of 2.18e9 elements each (4.4 GB), beyond 2^31: element
    # offsets of the last heads need 64-bit arithmetic in every pass (table,
    # preparation, forward, epilogue).  Inputs are drawn on the GPU from a
    # seeded generator; the oracle checks sampled rows of the first and last
    # heads.
    s, h, d = 32768 + 5, 520, 128
    assert s * h * d > 2 ** 31
    g = torch.Generator(device=DEV).manual_seed(11)
    q, k, v = (torch.randn((1, s, h, d), device=DEV, generator=g, dtype=torch.bfloat16)
               for _ in range(3))
    pos = np.random.default_rng(12).integers(0, 200, size=(s, 2)).astype(np.int32)
    rope = ja.rope_table_2d(torch.from_numpy(pos).to(DEV), d)
    _say(f"bf16 S={s} H={h} D={d}: {s * h * d / 2 ** 31:.3f} x 2^31 elements per tensor")
    out = ja.fwd_bf16(q, k, v, rope)
    torch.cuda.synchronize()
    heads = [0, h - 1]
    rows = np.unique(np.concatenate([np.random.default_rng(13).choice(s, 14, replace=False),
                                     [0, s - 1]]))
    qs, ks, vs = (t[:, :, heads].cpu() for t in (q, k, v))
    ref, _ = oracle.joint_attention(qs, ks, vs, pos, rows=rows)
    got = out[:, :, heads].cpu()[:, rows]
    _say(f"  rel_l2={rel_l2(got, ref):.3e} max_abs={max_abs(got, ref):.3e}")
    assert rel_l2(got, ref) <= BF16_REL_L2 and max_abs(got, ref) <= BF16_MAX_ABS
