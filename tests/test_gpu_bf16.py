"""GPU parity of the RoPE table and the BF16 joint-attention forward against
the fp64 oracle (calls go through the C ABI via the Python binding): outputs
within the stated tolerances, the rotated K bit for bit (both sides round
the fp64 rotation once to bf16)."""
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
    """The one-call forward: positions in, the library builds the table."""
    qd, kd, vd = (t.to(DEV) for t in (q, k, v))
    out = ja.fwd_bf16(qd, kd, vd, pos, theta, **kw)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("name,d", [("tiny", 64), ("t2i_2048", 128), ("i2i_2048", 128)])
def test_rope_table_matches_fp64_cos_sin(name, d):
    # the fp64 table against cos/sin of the oracle's angles (the device's
    # pow and sincos may differ from the host's in the last bit)
    w = synth.WORKLOADS[name].replace(head_dim=d)
    pos = synth.positions(w)
    _say(f"rope table {name} D={d} S={w.seq_len}")
    got = ja.rope_table_2d(torch.from_numpy(pos).to(DEV), d).cpu().numpy()
    ang = oracle.rope_angles(pos, d)
    ref = np.stack([np.cos(ang), np.sin(ang)], axis=-1)
    assert got.dtype == np.float64 and got.shape == ref.shape
    # a few ulps of the angle (up to ~390 rad) and of cos/sin
    np.testing.assert_allclose(got, ref, rtol=0, atol=4e-14)
    # tokens at (0, 0) (the text) are not rotated: cos 1 and sin 0 exactly
    origin = (pos == 0).all(axis=1)
    assert np.all(got[origin, :, 0] == 1.0) and np.all(got[origin, :, 1] == 0.0)


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


@pytest.mark.parametrize("s,d,b,h,rope", [(1, 64, 4, 64, True), (65, 128, 4, 64, True),
                                          (700, 128, 2, 64, True), (1037, 64, 2, 64, True),
                                          (520, 128, 2, 64, False)])
def test_ragged_lengths_wide_shape(s, d, b, h, rope):
    # Enough (512-query block, head, batch row) items to fill the CUs, so the
    # forward runs its wide shape (eight 64-row waves per workgroup) on
    # ragged lengths, with and without RoPE; the shapes above, whose wide
    # items would fill at most half of the CUs, run the small one (four
    # 32-row waves).
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    assert -(-s // 512) * h * b >= n_cu
    w = synth.Workload("ragged_wide", b, h, d, n_text=s, grid=0, outlier_frac=0.02)
    q, k, v, _ = synth.make_qkv(w, seed=s)
    rng = np.random.default_rng(s)
    pos = rng.integers(0, 200, size=(s, 2)).astype(np.int32) if rope else None
    _say(f"bf16 ragged wide S={s} D={d} B={b} H={h} rope={rope}")
    out, lse = _run_bf16(q, k, v, pos, return_lse=True)
    ref, ref_lse = oracle.joint_attention(q, k, v, pos)
    assert rel_l2(out, ref) <= BF16_REL_L2
    assert row_scaled_max_abs(out, ref) <= BF16_MAX_ABS
    assert max_abs(lse, ref_lse) <= 1e-2


@pytest.mark.parametrize("b,h", [(4, 64), (1, 2)])
def test_running_max_growth_across_tiles(b, h):
    # Scores built so that a row's running max climbs by about 56 (exp2
    # domain) per 32-key tile (query magnitude 64 on a key ramp over
    # [-64, 64]), by 28 or 14 per tile (32, 16: the max moves every few
    # tiles, P up to the rescale threshold in between), or sits at the first
    # key (negative magnitudes): the rescale path of the forward, in the wide
    # shape (4 x 64 heads) and the small one (2 heads), no RoPE.
    s, d = 600, 128
    rng = np.random.default_rng(11)
    q = 0.05 * rng.standard_normal((b, s, h, d))
    k = 0.05 * rng.standard_normal((b, s, h, d))
    v = rng.standard_normal((b, s, h, d))
    mags = np.array([64.0, 32.0, 16.0, 8.0, -64.0, -8.0, 0.0, 1.0])
    q[..., 0] = mags[np.arange(s) % len(mags)][None, :, None]
    k[..., 0] = np.linspace(-64.0, 64.0, s)[None, :, None]
    q, k, v = (torch.from_numpy(t.astype(np.float32)).to(torch.bfloat16) for t in (q, k, v))
    _say(f"bf16 running-max growth S={s} D={d} B={b} H={h}")
    out, lse = _run_bf16(q, k, v, None, return_lse=True)
    ref, ref_lse = oracle.joint_attention(q, k, v, None)
    assert torch.isfinite(out.float()).all()
    assert rel_l2(out, ref) <= BF16_REL_L2
    assert row_scaled_max_abs(out, ref) <= BF16_MAX_ABS
    assert max_abs(lse, ref_lse) <= 1e-2


def test_rope_base_500():
    # another RoPE base than the default, through the one-call forward (its
    # table built from the positions) and the preparation pass (rotated K
    # bit for bit)
    w = synth.Workload("theta500", 2, 3, 128, n_text=77, grid=11, outlier_frac=0.03)
    q, k, v, _ = synth.make_qkv(w, 4)
    pos = synth.positions(w)
    _say("bf16 theta=500")
    out = _run_bf16(q, k, v, pos, theta=500.0)
    ref, _ = oracle.joint_attention(q, k, v, pos, theta=500.0)
    assert rel_l2(out, ref) <= BF16_REL_L2
    assert row_scaled_max_abs(out, ref) <= BF16_MAX_ABS
    ref_default, _ = oracle.joint_attention(q, k, v, pos)
    assert rel_l2(out, ref_default) > 10 * BF16_REL_L2    # the base matters here
    kv = ja.prep_kv_bf16(k.to(DEV), v.to(DEV), pos, 500.0).cpu()
    s_pad = (w.seq_len + 63) // 64 * 64
    kr = kv[: 2 * 2 * 3 * s_pad * 128].view(torch.bfloat16).view(2, 3, s_pad, 128)
    kref = oracle.rotated_qk(k, pos, theta=500.0).to(torch.bfloat16)
    assert torch.equal(kr[:, :, :w.seq_len].view(torch.int16),
                       kref.permute(0, 2, 1, 3).contiguous().view(torch.int16))


@pytest.mark.parametrize("lo,hi", [(0, 300), (-40, 3000), (1024, 5000)])
def test_positions_path_equals_table_path(lo, hi):
    # The forward given positions reads Q's cos/sin from the coordinate table
    # when a wave's coordinates all lie in [0, 1024), else from the per-token
    # table; either way the output equals the one from a prebuilt per-token
    # table bit for bit.  (-40, 3000): waves of both kinds; (1024, 5000):
    # none inside.
    w = synth.Workload("coords", 1, 64, 128, n_text=1100, grid=0, outlier_frac=0.01)
    q, k, v, _ = synth.make_qkv(w, 13)
    pos = np.random.default_rng(lo + 77).integers(lo, hi, size=(w.seq_len, 2)).astype(np.int32)
    if lo == -40:
        pos[:600] = np.abs(pos[:600]) % 1024            # the first waves inside
    _say(f"bf16 positions path vs table path, coordinates in [{lo}, {hi})")
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    pos_d = torch.from_numpy(pos).to(DEV)
    out_pos, lse_pos = ja.fwd_bf16(qd, kd, vd, pos_d, return_lse=True)
    out_tab, lse_tab = ja.fwd_bf16(qd, kd, vd, rope=ja.rope_table_2d(pos_d, 128),
                                   return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(out_pos.view(torch.int16), out_tab.view(torch.int16))
    assert torch.equal(lse_pos, lse_tab)
    rows = np.unique(np.concatenate([np.arange(0, w.seq_len, 37), [w.seq_len - 1]]))
    ref, _ = oracle.joint_attention(q, k, v, pos, rows=rows)
    got = out_pos.cpu()[:, rows]
    assert rel_l2(got, ref) <= BF16_REL_L2
    assert row_scaled_max_abs(got, ref) <= BF16_MAX_ABS


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
    ja.fwd_bf16(qd, kd, vd, rope=rope, out=out)
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
        ja.fwd_bf16(qd, kd, vd, rope=rope, out=o)
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


@pytest.mark.parametrize("heads", [6, 3])
def test_sequence_parallel_shard_shapes(heads):
    # The per-GPU share of 16896 tokens under sequence parallelism over 4 or
    # 8 GPUs: all tokens, 24/u heads.  Six heads give 198 wide items (the
    # wide shape, one partial round); three give 99, which the small shape
    # (396 items of 128 rows) covers.
    w = synth.WORKLOADS["t2i_2048"].replace(heads=heads)
    q, k, v, idx, pos = _gpu_inputs(w, 7)
    rows = sample_rows(w.seq_len, w.n_text, idx, 128, seed=heads)
    _say(f"bf16 shard shape S={w.seq_len} H={heads} sampled rows={len(rows)}")
    out, lse = _run_bf16(q, k, v, pos, return_lse=True)
    ref, ref_lse = oracle.joint_attention(q, k, v, pos, rows=rows)
    got, got_lse = out.cpu()[:, rows], lse.cpu()[:, :, rows]
    _say(f"  rel_l2={rel_l2(got, ref):.3e}")
    assert rel_l2(got, ref) <= BF16_REL_L2
    assert row_scaled_max_abs(got, ref) <= BF16_MAX_ABS
    assert max_abs(got_lse, ref_lse) <= 2e-2


def test_split_last_round_parity():
    # A shape whose last round of workgroups is mostly idle, so the forward
    # splits those work items over key ranges and merges them (the items of
    # the last head's upper query blocks).  Checked against the oracle on
    # rows of split items and of whole items, and against the unsplit launch.
    base = synth.WORKLOADS["t2i_1024"]
    w = ws = None
    for heads in range(8, 65):   # first head count for which a split is planned
        w = base.replace(heads=heads)
        ws = (ja.fwd_bf16_workspace_bytes(w.batch, w.seq_len, heads, 128)
              - ja.fwd_bf16_workspace_bytes(w.batch, w.seq_len, heads, 128, split=False))
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


def test_split_round_mixing_whole_and_leftover_query_blocks():
    # 16500 tokens make 33 query blocks of 512 rows per head, the last one
    # partial (116 rows).  The work items are the first 32 blocks of every
    # head, head by head, then the 33rd block of every head; with 26 heads on
    # 256 CUs the last round (90 items, split over key ranges) holds the
    # first 32 blocks of heads 24 and 25 and all 26 partial blocks.  Sampled
    # rows cover early blocks, the split heads and the partial last block;
    # the unsplit launch is the second reference.
    w = synth.Workload("mixed_split", 1, 26, 128, n_text=116, grid=128, outlier_frac=0.01)
    ws = (ja.fwd_bf16_workspace_bytes(1, w.seq_len, w.heads, 128)
          - ja.fwd_bf16_workspace_bytes(1, w.seq_len, w.heads, 128, split=False))
    q, k, v, idx, pos = _gpu_inputs(w, 11)
    _say(f"bf16 mixed split round: S={w.seq_len} H={w.heads} workspace={ws} B")
    out, lse = _run_bf16(q, k, v, pos, return_lse=True)
    out_ns, lse_ns = _run_bf16(q, k, v, pos, return_lse=True, split=False)
    rows = np.unique(np.concatenate([sample_rows(w.seq_len, w.n_text, idx, 96, seed=3),
                                     np.arange(16384, w.seq_len, 5), [15871, 15872, 16383]]))
    ref, ref_lse = oracle.joint_attention(q, k, v, pos, rows=rows)
    got, got_lse = out.cpu()[:, rows], lse.cpu()[:, :, rows]
    _say(f"  rel_l2={rel_l2(got, ref):.3e} vs unsplit {rel_l2(out.cpu(), out_ns.cpu()):.3e}")
    assert rel_l2(got, ref) <= BF16_REL_L2
    assert row_scaled_max_abs(got, ref) <= BF16_MAX_ABS
    assert max_abs(got_lse, ref_lse) <= 2e-2
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
    # V transposed in 32-key tiles in the documented key order; padding is
    # zero
    w = synth.Workload("prep", 2, h, d, n_text=s, grid=0)
    q, k, v, _ = synth.make_qkv(w, seed=21)
    pos = np.random.default_rng(s).integers(0, 300, size=(s, 2)).astype(np.int32)
    if strided:
        kd, vd = (t.permute(0, 2, 1, 3).contiguous().to(DEV).permute(0, 2, 1, 3) for t in (k, v))
    else:
        kd, vd = k.to(DEV), v.to(DEV)
    rope = ja.rope_table_2d(torch.from_numpy(pos).to(DEV), d)
    _say(f"prep kv S={s} D={d} H={h} strided={strided}")
    kv = ja.prep_kv_bf16(kd, vd, rope=rope).cpu()
    # with positions only, the table the call builds follows K and V^T
    kv_pos = ja.prep_kv_bf16(kd, vd, pos).cpu()
    s_pad = (s + 63) // 64 * 64
    n = 2 * h * s_pad * d
    kr = kv[: 2 * n].view(torch.bfloat16).view(2, h, s_pad, d)
    vt = kv[2 * n:4 * n].view(torch.bfloat16).view(2, h, s_pad // 32, d, 32)
    assert torch.equal(kv_pos[:kv.numel()], kv)
    table = kv_pos[kv.numel():kv.numel() + s * d * 8].numpy().view(np.float64)
    assert np.array_equal(table, rope.cpu().numpy().ravel())
    # then the coordinate table: (cos, sin) of c * w_k for c < 1024, whose
    # entries equal the per-token table's bit for bit (pairs below D/4 by
    # the token's row, the others by its column)
    align = lambda x: (x + 255) // 256 * 256
    c0 = kv.numel() + align(s * d * 8)
    assert kv_pos.numel() == c0 + align(1024 * (d // 4) * 16)
    ctab = kv_pos[c0:c0 + 1024 * (d // 4) * 16].numpy().view(np.float64).reshape(1024, d // 4, 2)
    tab = table.reshape(s, d // 2, 2)
    assert np.array_equal(tab[:, :d // 4].view(np.uint64), ctab[pos[:, 0]].view(np.uint64))
    assert np.array_equal(tab[:, d // 4:].view(np.uint64), ctab[pos[:, 1]].view(np.uint64))
    kref = oracle.rotated_qk(k, pos).to(torch.bfloat16)
    assert torch.equal(kr[:, :, :s].view(torch.int16), kref.permute(0, 2, 1, 3).contiguous().view(torch.int16))
    assert not kr[:, :, s:].view(torch.int16).any()
    order = torch.tensor([16 * (j // 16) + _slot_key(j % 16) for j in range(s_pad)])
    vpad = torch.zeros((2, s_pad, h, d), dtype=torch.bfloat16)
    vpad[:, :s] = v
    vref = vpad[:, order].permute(0, 2, 3, 1)            # [B, H, D, S_pad]
    vref = vref.reshape(2, h, d, s_pad // 32, 32).permute(0, 1, 3, 2, 4)   # 32-key tiles
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
    _say(f"bf16 S={s} H={h} D={d}: {s * h * d / 2 ** 31:.3f} x 2^31 elements per tensor")
    out = ja.fwd_bf16(q, k, v, pos)
    torch.cuda.synchronize()
    heads = [0, h - 1]
    rows = np.unique(np.concatenate([np.random.default_rng(13).choice(s, 14, replace=False),
                                     [0, s - 1]]))
    qs, ks, vs = (t[:, :, heads].cpu() for t in (q, k, v))
    ref, _ = oracle.joint_attention(qs, ks, vs, pos, rows=rows)
    got = out[:, :, heads].cpu()[:, rows]
    _say(f"  rel_l2={rel_l2(got, ref):.3e} max_abs={max_abs(got, ref):.3e}")
    assert rel_l2(got, ref) <= BF16_REL_L2 and max_abs(got, ref) <= BF16_MAX_ABS
