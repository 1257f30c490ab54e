"""Dense joint attention, fp64 (oracle; test infrastructure only).

Joint attention ("Speed Up Image Generation with FLUX 3 Image Klein on NVIDIA
Blackwell GPUs", section "FLUX 3 inference with TensorRT LLM VisualGen"): the
text, noisy-target and reference-image tokens form one sequence and every
query attends to every key of it, with no mask.  Per batch row b and head h

    O[b, i, h] = sum_j softmax_j(Q[b,i,h] . K[b,j,h] / sqrt(D)) V[b, j, h]
    LSE[b, h, i] = log sum_j exp(Q[b,i,h] . K[b,j,h] / sqrt(D))

Written as the textbook definition: scores, max-shifted exponentials,
normalisation.  Query rows are independent, so `rows` evaluates just those
rows exactly (used for spot checks at full size); chunking over query rows is
only there to bound memory and changes nothing in the arithmetic of a row.
"""
from __future__ import annotations

import math

import numpy as np
import torch

from .bf16 import bf16_round
from .norm import prologue

_CHUNK = 2048


def attention(q, k, v, scale: float | None = None, rows=None):
    """softmax(Q K^T * scale) V in fp64.

    q, k, v: [B, S, H, D] tensors of any float dtype (converted exactly to
    fp64).  scale defaults to 1/sqrt(D).  rows: optional 1-D index array of
    query rows to evaluate.  Returns (O [B, R, H, D] fp64, LSE [B, H, R] fp64)
    where R = S or len(rows).
    """
    q = torch.as_tensor(q).to(torch.float64)
    k = torch.as_tensor(k).to(torch.float64)
    v = torch.as_tensor(v).to(torch.float64)
    b, s, h, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if rows is not None:
        q = q[:, torch.as_tensor(np.asarray(rows), dtype=torch.int64)]
    r = q.shape[1]
    o = torch.empty((b, r, h, d), dtype=torch.float64)
    lse = torch.empty((b, h, r), dtype=torch.float64)
    for bi in range(b):
        for hi in range(h):
            kt = k[bi, :, hi, :].T.contiguous()            # [D, S]
            vb = v[bi, :, hi, :].contiguous()              # [S, D]
            for c0 in range(0, r, _CHUNK):
                qc = q[bi, c0:c0 + _CHUNK, hi, :]          # [c, D]
                sc = (qc @ kt) * scale                     # [c, S]
                m = sc.max(dim=1, keepdim=True).values
                p = torch.exp(sc - m)
                l = p.sum(dim=1, keepdim=True)
                o[bi, c0:c0 + _CHUNK, hi, :] = (p @ vb) / l
                lse[bi, hi, c0:c0 + _CHUNK] = (m + torch.log(l))[:, 0]
    return o, lse


def rotated_qk(x, pos=None, theta: float = 10000.0, norm_g=None, eps: float = 1e-6,
               round_bf16: bool = True) -> torch.Tensor:
    """Q or K as attention consumes it: the epilogue's RMSNorm (weight norm_g,
    if given) and RoPE (if pos is given) in fp64, then, with round_bf16,
    ONE rounding to bf16 (round to nearest even), because the pages place
    both in the QKV projection's epilogue, whose output is stored in the
    model's working precision before attention reads it.  With neither norm
    nor RoPE the bf16 input is returned unchanged.  Returns fp64."""
    x = torch.as_tensor(x)
    if norm_g is None and pos is None:
        return x.to(torch.float64)
    y = prologue(x, pos, theta, norm_g, eps)
    return bf16_round(y) if round_bf16 else y


def joint_attention(q, k, v, pos=None, theta: float = 10000.0,
                    scale: float | None = None, round_rotated: bool = True,
                    rows=None, norm=None):
    """The bf16 hot path's reference: RoPE on Q and K, then attention.

    Q and K are normalized (norm=(g_q, g_k, eps), optional) and rotated
    (pos, optional) in fp64 and rounded once to bf16 (`rotated_qk`); with
    round_rotated=False they stay unrounded fp64, for information.
    Attention itself is fp64.  pos=None: no RoPE.
    """
    g_q, g_k, eps = norm if norm is not None else (None, None, 1e-6)
    q = rotated_qk(q, pos, theta, g_q, eps, round_rotated)
    k = rotated_qk(k, pos, theta, g_k, eps, round_rotated)
    return attention(q, k, v, scale=scale, rows=rows)


def brute_force_attention(q, k, v, scale: float | None = None):
    """Pure-Python triple loop over (b, h, i); for tiny shapes only.

    Uses math.fsum so the reductions are exactly rounded; it is the
    independent check of the vectorised `attention`.  The key count may differ
    from the query count.
    """
    q = torch.as_tensor(q).to(torch.float64).tolist()
    k = torch.as_tensor(k).to(torch.float64).tolist()
    v = torch.as_tensor(v).to(torch.float64).tolist()
    b_n, s_n, h_n, d_n = len(q), len(q[0]), len(q[0][0]), len(q[0][0][0])
    sk_n = len(k[0])
    if scale is None:
        scale = 1.0 / math.sqrt(d_n)
    o = [[[[0.0] * d_n for _ in range(h_n)] for _ in range(s_n)] for _ in range(b_n)]
    lse = [[[0.0] * s_n for _ in range(h_n)] for _ in range(b_n)]
    for b in range(b_n):
        for h in range(h_n):
            for i in range(s_n):
                sc = [math.fsum(q[b][i][h][t] * k[b][j][h][t] for t in range(d_n)) * scale
                      for j in range(sk_n)]
                m = max(sc)
                e = [math.exp(x - m) for x in sc]
                z = math.fsum(e)
                for t in range(d_n):
                    o[b][i][h][t] = math.fsum(e[j] * v[b][j][h][t] for j in range(sk_n)) / z
                lse[b][h][i] = m + math.log(z)
    return torch.tensor(o, dtype=torch.float64), torch.tensor(lse, dtype=torch.float64)


# Block granularity of the block-sparse variant (queries x keys).
QUERY_BLOCK = 128
KEY_BLOCK = 64


def block_sparse_attention(q, k, v, mask, pos=None, theta: float = 10000.0,
                           scale: float | None = None, rows=None,
                           q_block: int = QUERY_BLOCK, k_block: int = KEY_BLOCK, norm=None):
    """Joint attention restricted by a block mask (the kernel half of the
    pages' block-sparse attention, section "Quantized and sparse attention":
    Sol-Attention runs on a general block-sparse attention kernel; how its
    blocks are chosen is not on the pages, so the mask is an input here).

    mask: [B, H, ceil(S / q_block), ceil(S / k_block)], nonzero = computed.
    Query i attends key j iff mask[b, h, i // q_block, j // k_block] != 0;
    the softmax runs over the attended keys only.  A query row with no
    attended key gets O = 0 and LSE = -inf.  The Q/K prologue and its bf16
    rounding are those of `joint_attention`; attention itself is fp64.
    Returns (O [B, R, H, D] fp64, LSE [B, H, R] fp64).
    """
    g_q, g_k, eps = norm if norm is not None else (None, None, 1e-6)
    q = rotated_qk(q, pos, theta, g_q, eps)
    k = rotated_qk(k, pos, theta, g_k, eps)
    v = torch.as_tensor(v).to(torch.float64)
    mask = torch.as_tensor(np.asarray(mask)) != 0
    b, s, h, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    rows = np.arange(s) if rows is None else np.asarray(rows)
    key_blk = torch.arange(s) // k_block
    o = torch.zeros((b, len(rows), h, d), dtype=torch.float64)
    lse = torch.full((b, h, len(rows)), -math.inf, dtype=torch.float64)
    for bi in range(b):
        for hi in range(h):
            kt = k[bi, :, hi, :].T.contiguous()
            vb = v[bi, :, hi, :].contiguous()
            for c0 in range(0, len(rows), _CHUNK):
                r = torch.as_tensor(rows[c0:c0 + _CHUNK], dtype=torch.int64)
                allowed = mask[bi, hi][(r // q_block)[:, None], key_blk[None, :]]   # [c, S]
                sc = (q[bi, r, hi, :] @ kt) * scale
                sc = torch.where(allowed, sc, torch.tensor(-math.inf, dtype=torch.float64))
                m = sc.max(dim=1, keepdim=True).values
                live = torch.isfinite(m[:, 0])
                p = torch.where(allowed, torch.exp(sc - torch.where(torch.isfinite(m), m, 0.0)), 0.0)
                l = p.sum(dim=1, keepdim=True)
                oc = (p @ vb) / torch.where(l > 0, l, 1.0)
                o[bi, c0:c0 + len(r), hi, :] = torch.where(live[:, None], oc, 0.0)
                lse[bi, hi, c0:c0 + len(r)] = torch.where(live, (m + torch.log(l))[:, 0],
                                                          torch.tensor(-math.inf, dtype=torch.float64))
    return o, lse
