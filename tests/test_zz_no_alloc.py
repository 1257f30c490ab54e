"""The no-allocation BF16 forward (joint_attn_fwd_bf16_prepared_noalloc)
against the forward it varies, joint_attn_fwd_bf16_prepared: the same
kernels and split plan, with the split's partial results in the library's
static scratch instead of a workspace.  Two calls in a row, the second on a
smaller input (the scratch still holds the first call's partials), on shapes
whose last round of workgroups is split, so the scratch is used."""
import numpy as np
import pytest
import torch

import joint_attention_attn_amd as ja
import oracle
import synth
from parity_util import BF16_REL_L2, BF16_MAX_ABS, rel_l2, row_scaled_max_abs

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _split_heads(s, d):
    """The first head count at which the forward splits its last round."""
    for h in range(2, 200):
        if ja.fwd_bf16_workspace_bytes(1, s, h, d) > ja.fwd_bf16_workspace_bytes(1, s, h, d,
                                                                                 split=False):
            return h
    raise AssertionError(f"no split planned at S={s} D={d}")


def test_noalloc_matches_the_workspace_forward_on_two_calls():
    for s, d, seed in ((4608, 128, 1), (2000, 64, 2)):        # the second call is smaller
        h = _split_heads(s, d)
        w = synth.Workload("noalloc", 1, h, d, n_text=s, grid=0, outlier_frac=0.01)
        q, k, v, idx = synth.make_qkv(w, seed)
        pos = np.random.default_rng(seed).integers(0, 128, size=(s, 2)).astype(np.int32)
        print(f"noalloc S={s} H={h} D={d}", flush=True)
        qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
        rope = ja.rope_table_2d(torch.from_numpy(pos).to(DEV), d)
        kv = ja.prep_kv_bf16(kd, vd, rope=rope)
        ref, ref_lse = ja.fwd_bf16_prepared(qd, kv, rope=rope, return_lse=True)
        out = torch.full(q.shape, float("nan"), dtype=torch.bfloat16, device=DEV)
        got, lse = ja.fwd_bf16_prepared_noalloc(qd, kv, rope=rope, out=out, return_lse=True)
        torch.cuda.synchronize()
        assert got is out
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
        assert torch.equal(lse, ref_lse)
        # and the oracle on rows of the split items (the last head's last rows)
        rows = np.unique(np.concatenate([np.arange(s - 16, s), [0, 1, s // 2]]))
        want, _ = oracle.joint_attention(q, k, v, pos, rows=rows)
        part = out.cpu()[:, rows]
        assert rel_l2(part, want) <= BF16_REL_L2
        assert row_scaled_max_abs(part, want) <= BF16_MAX_ABS


def test_noalloc_rejects_before_launch():
    # invalid calls are refused on the host, before anything is launched
    w = synth.Workload("noalloc_bad", 1, 2, 64, n_text=100, grid=0)
    q, k, v, _ = synth.make_qkv(w, 3)
    qd = q.to(DEV)
    kv = ja.prep_kv_bf16(k.to(DEV), v.to(DEV))
    lib = ja.load()
    assert lib.joint_attn_fwd_bf16_prepared_noalloc(None, None, None, 0, None, None,
                                                    None) == ja.JA_ERR_INVALID_ARG
    with pytest.raises(ja.JointAttnError):
        ja.fwd_bf16_prepared_noalloc(qd, kv[:1024])          # prepared buffer too small
