"""FP8 (OCP e4m3fn) quantization of rotated Q/K and V, and the FP8 attention
reference (oracle; test infrastructure only).

The pages enable FP8 attention by setting qk_dtype and v_dtype to fp8 ("Speed
Up Image Generation with FLUX 3 Image Klein on NVIDIA Blackwell GPUs", section
"Quantized and sparse attention") and state nothing else.  Readings taken:

* format: OCP 8-bit floating point E4M3 ("fn": bias 7, no infinities, largest
  finite magnitude 448, subnormal spacing 2^-9), round to nearest even,
  saturating to +-448;
* granularity: one fp32 scale per (batch, token, head) over the D elements of
  that head vector ("per token"), scale = amax / 448, and scale = 1 when the
  vector is all zeros; Q and K are quantized after RoPE, V as given;
* precision of the decision: the quantizer rounds values that were computed
  in fp32 with a fixed operation order (`oracle.rope.rotate_fp32`, then
  fl(x / scale)), so the codes it produces are a deterministic function of
  the inputs that any fp32 implementation with the same order reproduces bit
  for bit.

The attention reference for this path is plain fp64 attention on the
dequantized tensors (code value x scale), with no further RoPE.
"""
from __future__ import annotations

import numpy as np
import torch

from .attention import attention
from .rope import rope_table_fp32, rotate_fp32

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


def _quantize_rows(r: np.ndarray):
    """Per-(b, s, h) e4m3 quantization of fp32 r [B, S, H, D].

    amax = max |r| over D; scale = fl32(amax / 448) (1 when amax = 0);
    code = e4m3(clamp(fl32(r / scale), -448, 448)).  Returns (uint8 codes
    [B, S, H, D], fp32 scales [B, H, S]).
    """
    amax = np.max(np.abs(r), axis=-1)                                   # fp32 exact
    scale = (amax / np.float32(E4M3_MAX)).astype(np.float32)
    scale = np.where(amax == 0, np.float32(1.0), scale).astype(np.float32)
    y = (r / scale[..., None]).astype(np.float32)
    y = np.clip(y, np.float32(-E4M3_MAX), np.float32(E4M3_MAX))
    codes = e4m3_encode(e4m3_round(y))
    return codes, np.ascontiguousarray(np.transpose(scale, (0, 2, 1)))


def quant_rope_fp8(q, k, v, pos, theta: float = 10000.0):
    """RoPE on Q and K (fp32, `rotate_fp32` order), then per-token e4m3 quantization
    of Q, K and V.  Returns (q8, k8, v8, sq, sk, sv): uint8 codes
    [B, S, H, D] and fp32 scales [B, H, S].  pos=None skips the rotation."""
    q = torch.as_tensor(q).to(torch.float32).numpy()
    k = torch.as_tensor(k).to(torch.float32).numpy()
    v = torch.as_tensor(v).to(torch.float32).numpy()
    if pos is not None:
        table = rope_table_fp32(pos, q.shape[-1], theta)
        q = rotate_fp32(q, table)
        k = rotate_fp32(k, table)
    q8, sq = _quantize_rows(q)
    k8, sk = _quantize_rows(k)
    v8, sv = _quantize_rows(v)
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
