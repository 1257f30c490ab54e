"""FP8 (OCP e4m3fn) quantization of rotated Q/K and V, and the FP8 attention
reference (oracle; test infrastructure only).

The pages enable FP8 attention by setting qk_dtype and v_dtype to fp8 ("Speed
Up Image Generation with FLUX 3 Image Klein on NVIDIA Blackwell GPUs", section
"Quantized and sparse attention") and state nothing else.  Readings taken:

* format: OCP 8-bit floating point E4M3 ("fn": bias 7, no infinities, largest
  finite magnitude 448, subnormal spacing 2^-9), round to nearest even,
  saturating to +-448;
* granularity: one fp32 scale per (batch, token, head) over the D elements of
  that head vector ("per token"), scale = 1 when the vector is all zeros;
  Q and K are quantized after RoPE, V as given;
* scale value: for V, amax / 448 (the largest element lands on 448); for Q
  and K, the smallest power of two s with amax <= 448 s (at least 2^-126, the
  smallest normal fp32 power of two).  A power of two is the OCP microscaling
  convention for shared scales (an E8M0 exponent): the matrix cores apply it
  exactly to the Q K^T product, and x / s is exact.  e4m3 is a floating-point
  format, so its relative precision does not depend on where amax lands in
  (224, 448];
* precision: the rotated (and normalized) Q/K come from the fp64 prologue
  of `oracle.norm.prologue` with no intermediate rounding; amax is taken in
  fp64; the V scale is stored as fp32 (fl32(amax / 448)); the code is the
  e4m3 rounding of x / scale evaluated in fp64.

The attention reference for this path is plain fp64 attention on the
dequantized tensors (code value x scale), with no further RoPE.
"""
from __future__ import annotations

import numpy as np
import torch

from .attention import attention
from .bf16 import bf16_round
from .norm import prologue

E4M3_MAX = 448.0


def e4m3_round(x) -> np.ndarray:
    """Round to the nearest e4m3fn value (ties to even), saturating at 448.

    Returns the rounded values as fp64.  Normal numbers 2^e * 1.mmm have
    e >= -6 and three fraction bits, so their spacing is 2^(e-3); below 2^-6
    the subnormal spacing is 2^-9 = 2^(-6-3).
    """
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), E4M3_MAX)
    _, e = np.frexp(a)                   # a = f * 2^e with f in [0.5, 1)
    e = np.maximum(e - 1, -6)            # exponent of the leading bit, >= -6
    step = np.ldexp(1.0, e - 3)
    r = np.round(a / step) * step        # a/step is exact; np.round is half-even
    return np.copysign(r, x)


def e4m3_encode(r) -> np.ndarray:
    """Bit pattern (uint8) of values that are already e4m3fn-representable."""
    r = np.asarray(r, dtype=np.float64)
    sign = np.signbit(r).astype(np.uint8) << 7
    a = np.abs(r)
    _, e = np.frexp(a)
    e = e - 1
    normal = a >= 2.0 ** -6
    exp_field = np.where(normal, e + 7, 0).astype(np.int64)
    frac = np.where(normal, (a / np.ldexp(1.0, np.where(normal, e, 0)) - 1.0) * 8.0,
                    a * 512.0)
    frac_i = np.rint(frac).astype(np.int64)
    if not np.array_equal(frac_i, frac):
        raise ValueError("value is not representable in e4m3fn")
    return (sign | ((exp_field << 3) | frac_i).astype(np.uint8)).astype(np.uint8)


def e4m3_decode(code) -> np.ndarray:
    """Value (fp64) of e4m3fn bit patterns; 0x7F / 0xFF decode to NaN."""
    c = np.asarray(code, dtype=np.uint8).astype(np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    ef = (c >> 3) & 0xF
    m = c & 0x7
    val = np.where(ef == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.ldexp(1.0, ef - 7))
    val = np.where((ef == 15) & (m == 7), np.nan, val)
    return s * val


def pow2_scale(amax) -> np.ndarray:
    """Smallest power of two s with amax <= 448 s, as fp32 (1 when amax = 0,
    at least 2^-126).  With amax = f 2^x, f in [0.5, 1): 448 = 0.875 2^9, so
    s = 2^(x - 9) when f <= 0.875 and 2^(x - 8) otherwise.  amax may be fp32
    or fp64."""
    amax = np.asarray(amax)
    f, x = np.frexp(amax.astype(np.float64))
    k = np.maximum(x - 9 + (f > 0.875), -126)
    s = np.ldexp(np.float64(1.0), k).astype(np.float32)
    return np.where(amax == 0, np.float32(1.0), s).astype(np.float32)


def _quantize_rows(r, pow2: bool = False):
    """Per-(b, s, h) e4m3 quantization of r [B, S, H, D] (fp64 values).

    amax = max |r| over D; scale = pow2_scale(amax) when pow2, else
    fl32(amax / 448) (the fp32 number that is stored); 1 when amax = 0 either
    way.  code = e4m3(clamp(r / scale, -448, 448)) with r / scale in fp64.
    Returns (uint8 codes [B, S, H, D], fp32 scales [B, H, S]).
    """
    r = np.asarray(r, np.float64)
    amax = np.max(np.abs(r), axis=-1)
    if pow2:
        scale = pow2_scale(amax)
    else:
        # V is bf16: amax / 448 = (m / 7) 2^k has a period-3 binary expansion,
        # so its fp64 value never lands on an fp32 midpoint and the cast is
        # the correctly rounded fp32 quotient
        scale = (amax / E4M3_MAX).astype(np.float32)
        scale = np.where(amax == 0, np.float32(1.0), scale).astype(np.float32)
    y = np.clip(r / scale.astype(np.float64)[..., None], -E4M3_MAX, E4M3_MAX)
    codes = e4m3_encode(e4m3_round(y))
    return codes, np.ascontiguousarray(np.transpose(scale, (0, 2, 1)))


def quant_rope_fp8(q, k, v, pos, theta: float = 10000.0, norm=None):
    """RoPE on Q and K (after the optional RMS norm, all in fp64: the
    epilogue's `prologue`), then per-token e4m3 quantization of Q, K
    (power-of-two scales) and V (amax / 448).  Returns (q8, k8, v8, sq, sk,
    sv): uint8 codes [B, S, H, D] and fp32 scales [B, H, S].  pos=None skips
    the rotation; norm=(g_q, g_k, eps) RMS-normalizes Q and K first."""
    g_q, g_k, eps = norm if norm is not None else (None, None, 1e-6)
    q64 = prologue(q, pos, theta, g_q, eps).numpy()
    k64 = prologue(k, pos, theta, g_k, eps).numpy()
    v64 = torch.as_tensor(v).to(torch.float64).numpy()
    q8, sq = _quantize_rows(q64, pow2=True)
    k8, sk = _quantize_rows(k64, pow2=True)
    v8, sv = _quantize_rows(v64)
    return q8, k8, v8, sq, sk, sv


def dequantize(codes, scales) -> torch.Tensor:
    """code value x its (b, s, h) scale, fp64 [B, S, H, D] (exact)."""
    vals = e4m3_decode(np.asarray(codes))
    sc = np.transpose(np.asarray(scales, dtype=np.float64), (0, 2, 1))[..., None]
    return torch.from_numpy(vals * sc)


def fp8_attention(q8, k8, v8, sq, sk, sv, scale=None, rows=None):
    """fp64 attention on the dequantized Q/K/V (RoPE already applied)."""
    return attention(dequantize(q8, sq), dequantize(k8, sk), dequantize(v8, sv),
                     scale=scale, rows=rows)


# ---------------------------------------------------------------------------
# Repair of the tokens with the largest quantization error (VC-Attention FP8)
#
# In the pages' VC-Attention FP8 setting a budget rho = 0.005
# (vc_repair_budget) sets the share of tokens that get a correction: the ones
# whose quantization error is largest (same page, section "Quantized and
# sparse attention").  The pages say nothing more about the mechanism.
# Reading taken:
#
# * a token's error, per (batch, head), is the max-abs quantization error of
#   its key plus that of its value: e = max_d |k - k^| + max_d |v - v^|, with
#   k the rotated key that was quantized and k^ = code value * scale (all in
#   fp64); tokens are ranked by e rounded to fp32;
# * the ceil(rho * S) tokens with the largest e are repaired, ties to the
#   lower token index;
# * repairing a token adds its residual (k - k^, v - v^) back, i.e. the key
#   and value of that token enter attention at the precision of the bf16 path
#   (the rotated key rounded once to bf16, the bf16 value).  Queries stay FP8: a
#   query's error only affects its own row, a key's error every row.
# ---------------------------------------------------------------------------

def repair_count(budget: float, seq_len: int) -> int:
    """Repaired tokens per (batch, head): ceil(budget * seq_len)."""
    return int(np.ceil(np.float64(budget) * seq_len))


def _bshd_scales(scales) -> np.ndarray:
    return np.transpose(np.asarray(scales, dtype=np.float64), (0, 2, 1))[..., None]


def quant_error(x, codes, scales) -> np.ndarray:
    """max over D of |x - value(code) * scale| in fp64: float64 [B, H, S].
    x: the values that were quantized, [B, S, H, D]."""
    deq = e4m3_decode(codes) * _bshd_scales(scales)
    err = np.abs(np.asarray(x, np.float64) - deq)
    return np.ascontiguousarray(np.transpose(err.max(axis=-1), (0, 2, 1)))


def repair_errors(k, v, pos, k8, v8, sk, sv, theta: float = 10000.0, norm=None) -> np.ndarray:
    """Per-(b, h, token) error e = err(K) + err(V) in fp64, rounded to fp32 for
    the ranking: float32 [B, H, S] (K as the quantizer saw it: normalized
    with norm's g_k if given, rotated)."""
    k64 = prologue(k, pos, theta, norm[1] if norm is not None else None,
                   norm[2] if norm is not None else 1e-6).numpy()
    v64 = torch.as_tensor(v).to(torch.float64).numpy()
    return (quant_error(k64, k8, sk) + quant_error(v64, v8, sv)).astype(np.float32)


def repair_select(err, n: int) -> np.ndarray:
    """Token indices [B, H, n] (ascending) of the n largest errors of each
    (b, h) row; equal errors are taken in ascending token order."""
    err = np.asarray(err, np.float64)
    b, h, s = err.shape
    out = np.empty((b, h, n), dtype=np.int32)
    idx = np.arange(s)
    for bi in range(b):
        for hi in range(h):
            order = np.lexsort((idx, -err[bi, hi]))
            out[bi, hi] = np.sort(order[:n])
    return out


def repair_values(k, v, pos, idx, theta: float = 10000.0, norm=None):
    """Exact key and value of the repaired tokens: the rotated (and, with
    norm, normalized) key rounded once to bf16 as on the bf16 path, and the
    bf16 value, float64 [B, H, n, D]."""
    k64 = prologue(k, pos, theta, norm[1] if norm is not None else None,
                   norm[2] if norm is not None else 1e-6)
    kb = bf16_round(k64) if (pos is not None or norm is not None) else k64
    vb = torch.as_tensor(v).to(torch.float64)
    idx = np.asarray(idx)
    b, h, n = idx.shape
    d = kb.shape[-1]
    kr = torch.empty((b, h, n, d), dtype=torch.float64)
    vr = torch.empty((b, h, n, d), dtype=torch.float64)
    for bi in range(b):
        for hi in range(h):
            sel = torch.from_numpy(np.array(idx[bi, hi], dtype=np.int64))
            kr[bi, hi] = kb[bi, sel, hi]
            vr[bi, hi] = vb[bi, sel, hi]
    return kr, vr


def fp8_repaired_attention(q8, k8, v8, sq, sk, sv, idx, kr, vr, scale=None, rows=None):
    """fp64 attention on the dequantized Q/K/V in which the keys and values of
    the tokens idx[b, h] are replaced by their exact values kr / vr."""
    qd, kd, vd = dequantize(q8, sq), dequantize(k8, sk), dequantize(v8, sv)
    idx = np.asarray(idx)
    for bi in range(idx.shape[0]):
        for hi in range(idx.shape[1]):
            sel = torch.from_numpy(np.array(idx[bi, hi], dtype=np.int64))
            kd[bi, sel, hi] = torch.as_tensor(kr[bi, hi], dtype=torch.float64)
            vd[bi, sel, hi] = torch.as_tensor(vr[bi, hi], dtype=torch.float64)
    return attention(qd, kd, vd, scale=scale, rows=rows)
