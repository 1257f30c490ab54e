"""Python binding of libjoint_attn.so (MI355X joint text+image attention).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in include/joint_attn.h.  PyTorch supplies
device memory and the current stream.  There is no fallback: if the shared
library is missing or a call fails, a RuntimeError is raised.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

__all__ = [
    "JointAttnError", "library_path", "load", "rope_table_2d", "fwd_bf16",
    "fwd_bf16_workspace_bytes", "prep_kv_bf16", "fwd_bf16_prepared",
    "fwd_bf16_block_sparse_prepared", "Fp8Repair", "fp8_repair_plan", "repair_count",
    "quant_rope_fp8", "fwd_fp8", "Params", "fwd_bf16_block_sparse",
    "SPARSE_QUERY_BLOCK", "SPARSE_KEY_BLOCK", "block_mask_shape",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libjoint_attn.so")
_LIB = None

JA_OK, JA_ERR_INVALID_ARG, JA_ERR_UNSUPPORTED, JA_ERR_HIP = 0, 1, 2, 3
# block granularity of the block-sparse forward's mask (queries x keys)
SPARSE_QUERY_BLOCK, SPARSE_KEY_BLOCK = 128, 64


class JointAttnError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(what)


class Params(ctypes.Structure):
    """Mirror of ja_params."""
    _fields_ = [
        ("batch", ctypes.c_int32), ("seq_len", ctypes.c_int32),
        ("heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("q_sb", ctypes.c_int64), ("q_ss", ctypes.c_int64), ("q_sh", ctypes.c_int64),
        ("k_sb", ctypes.c_int64), ("k_ss", ctypes.c_int64), ("k_sh", ctypes.c_int64),
        ("v_sb", ctypes.c_int64), ("v_ss", ctypes.c_int64), ("v_sh", ctypes.c_int64),
        ("o_sb", ctypes.c_int64), ("o_ss", ctypes.c_int64), ("o_sh", ctypes.c_int64),
        ("softmax_scale", ctypes.c_float),
        ("q_norm", ctypes.c_void_p), ("k_norm", ctypes.c_void_p),
        ("norm_eps", ctypes.c_float),
    ]


class Fp8RepairC(ctypes.Structure):
    """Mirror of ja_fp8_repair."""
    _fields_ = [("n_rep", ctypes.c_int32), ("kbias", ctypes.c_void_p),
                ("kr", ctypes.c_void_p), ("vr", ctypes.c_void_p)]


def library_path() -> str:
    return _LIB_PATH


def load() -> ctypes.CDLL:
    """Load libjoint_attn.so (built by __graft_entry__.build()); raise if absent."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(
            f"{_LIB_PATH} is not built: run `python -c 'import __graft_entry__ as g; g.build()'`")
    lib = ctypes.CDLL(_LIB_PATH)
    vp, st = ctypes.c_void_p, ctypes.c_int
    pp = ctypes.POINTER(Params)
    lib.joint_attn_rope_table_2d.argtypes = [vp, ctypes.c_int32, ctypes.c_int32, ctypes.c_float, vp, vp]
    sz = ctypes.c_size_t
    lib.joint_attn_prep_kv_bf16_bytes.argtypes = [pp]
    lib.joint_attn_prep_kv_bf16_bytes.restype = sz
    lib.joint_attn_prep_kv_bf16.argtypes = [pp, vp, vp, vp, vp, sz, vp]
    lib.joint_attn_fwd_bf16.argtypes = [pp, vp, vp, sz, vp, vp, vp, vp, sz, vp]
    lib.joint_attn_fwd_bf16_block_sparse.argtypes = [pp, vp, vp, sz, vp, vp, vp, vp, vp, sz, vp]
    lib.joint_attn_fwd_bf16_workspace_bytes.argtypes = [pp]
    lib.joint_attn_fwd_bf16_workspace_bytes.restype = ctypes.c_size_t
    lib.joint_attn_quant_rope_fp8.argtypes = [pp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.joint_attn_prep_kv_fp8_bytes.argtypes = [pp]
    lib.joint_attn_prep_kv_fp8_bytes.restype = sz
    lib.joint_attn_prep_kv_fp8.argtypes = [pp, vp, vp, vp, vp, ctypes.POINTER(Fp8RepairC),
                                           vp, sz, vp]
    lib.joint_attn_fwd_fp8.argtypes = [pp, vp, vp, vp, sz, ctypes.POINTER(Fp8RepairC),
                                       vp, vp, vp, sz, vp]
    lib.joint_attn_fp8_repair_plan.argtypes = [pp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_int32,
                                               vp, vp, vp, vp, vp]
    lib.joint_attn_fp8_repair_plan.restype = st
    lib.joint_attn_fwd_fp8_workspace_bytes.argtypes = [pp]
    lib.joint_attn_fwd_fp8_workspace_bytes.restype = ctypes.c_size_t
    for fn in ("joint_attn_rope_table_2d", "joint_attn_prep_kv_bf16", "joint_attn_fwd_bf16",
               "joint_attn_fwd_bf16_block_sparse",
               "joint_attn_quant_rope_fp8", "joint_attn_prep_kv_fp8", "joint_attn_fwd_fp8"):
        getattr(lib, fn).restype = st
    lib.joint_attn_status_string.argtypes = [st]
    lib.joint_attn_status_string.restype = ctypes.c_char_p
    lib.joint_attn_last_error.argtypes = []
    lib.joint_attn_last_error.restype = ctypes.c_char_p
    _LIB = lib
    return lib


def _check(status: int, fn: str) -> None:
    if status != JA_OK:
        lib = load()
        msg = lib.joint_attn_status_string(status).decode()
        extra = lib.joint_attn_last_error().decode() if status == JA_ERR_HIP else ""
        raise JointAttnError(status, f"{fn}: {msg} {extra}".strip())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _bshd(t: torch.Tensor, name: str):
    if t.dim() != 4:
        raise ValueError(f"{name} must be 4-D [B, S, H, D], got {tuple(t.shape)}")
    if t.stride(3) != 1:
        raise ValueError(f"{name} must have a unit stride along D")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    return t.stride(0), t.stride(1), t.stride(2)


def _params(q, k, v, o, softmax_scale):
    b, s, h, d = q.shape
    for t, n in ((k, "k"), (v, "v"), (o, "out")):
        if tuple(t.shape) != (b, s, h, d):
            raise ValueError(f"{n} shape {tuple(t.shape)} != q shape {(b, s, h, d)}")
    p = Params(b, s, h, d)
    p.q_sb, p.q_ss, p.q_sh = _bshd(q, "q")
    p.k_sb, p.k_ss, p.k_sh = _bshd(k, "k")
    p.v_sb, p.v_ss, p.v_sh = _bshd(v, "v")
    p.o_sb, p.o_ss, p.o_sh = _bshd(o, "out")
    p.softmax_scale = float(softmax_scale or 0.0)
    return p


def _set_norm(p, q_norm=None, k_norm=None, norm_eps: float = 0.0):
    """Optional query/key RMS-norm weights: fp32 contiguous [head_dim] device
    tensors (None = that tensor is not normalized); norm_eps 0 = 1e-6."""
    for t, n in ((q_norm, "q_norm"), (k_norm, "k_norm")):
        if t is not None and (t.dtype != torch.float32 or t.dim() != 1 or not t.is_contiguous()
                              or t.numel() != p.head_dim or not t.is_cuda):
            raise ValueError(f"{n} must be a contiguous fp32 [{p.head_dim}] device tensor")
    p.q_norm = None if q_norm is None else q_norm.data_ptr()
    p.k_norm = None if k_norm is None else k_norm.data_ptr()
    p.norm_eps = float(norm_eps)
    return p


def rope_table_2d(pos: torch.Tensor, head_dim: int, theta: float = 10000.0) -> torch.Tensor:
    """(cos, sin) table [S, head_dim/2, 2] fp32 of 2D-axial RoPE for int32 pos [S, 2]."""
    if pos.dtype != torch.int32 or pos.dim() != 2 or pos.shape[1] != 2 or not pos.is_contiguous():
        raise ValueError("pos must be a contiguous int32 [S, 2] device tensor")
    table = torch.empty((pos.shape[0], head_dim // 2, 2), dtype=torch.float32, device=pos.device)
    st = load().joint_attn_rope_table_2d(_ptr(pos), pos.shape[0], head_dim, float(theta),
                                         _ptr(table), _stream(pos.device))
    _check(st, "joint_attn_rope_table_2d")
    return table


def _check_bf16(**tensors):
    for n, t in tensors.items():
        if t.dtype != torch.bfloat16:
            raise ValueError(f"{n} must be bfloat16")


def prep_kv_bf16(k, v, rope=None, k_norm=None, norm_eps: float = 0.0):
    """Prepared K/V buffer of the bf16 forward (uint8 device tensor): K
    RMS-normalized with weights `k_norm` (if given), rotated with `rope` (if
    given), V transposed."""
    _check_bf16(k=k, v=v)
    p = _set_norm(_params(k, k, v, k, 0.0), None, k_norm, norm_eps)
    lib = load()
    n = int(lib.joint_attn_prep_kv_bf16_bytes(ctypes.byref(p)))
    if n == 0:
        raise JointAttnError(JA_ERR_UNSUPPORTED, "joint_attn_prep_kv_bf16: unsupported shape")
    kv = torch.empty(n, dtype=torch.uint8, device=k.device)
    st = lib.joint_attn_prep_kv_bf16(ctypes.byref(p), _ptr(k), _ptr(v), _ptr(rope), _ptr(kv), n,
                                     _stream(k.device))
    _check(st, "joint_attn_prep_kv_bf16")
    return kv


def _fwd_prepared(fn, name, q, kv, rope, mask, softmax_scale, out, return_lse, split,
                  q_norm=None, norm_eps=0.0):
    _check_bf16(q=q)
    if kv.dtype != torch.uint8 or kv.dim() != 1 or kv.device != q.device:
        raise ValueError("kv must be the uint8 buffer from prep_kv_bf16 on q's device")
    if out is None:
        out = torch.empty(q.shape, dtype=torch.bfloat16, device=q.device)
    p = _set_norm(_params(q, q, q, out, softmax_scale), q_norm, None, norm_eps)
    lse = None
    if return_lse:
        lse = torch.empty((q.shape[0], q.shape[2], q.shape[1]), dtype=torch.float32, device=q.device)
    lib = load()
    ws_bytes = lib.joint_attn_fwd_bf16_workspace_bytes(ctypes.byref(p)) if split else 0
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device) if ws_bytes else None
    args = [ctypes.byref(p), _ptr(q), _ptr(kv), kv.numel(), _ptr(rope)]
    if mask is not None:
        args.append(_ptr(mask))
    st = fn(*args, _ptr(out), _ptr(lse), _ptr(ws), ws_bytes, _stream(q.device))
    _check(st, name)
    return (out, lse) if return_lse else out


def fwd_bf16_prepared(q, kv, rope=None, softmax_scale: float = 0.0, out=None,
                      return_lse: bool = False, split: bool = True, q_norm=None,
                      norm_eps: float = 0.0):
    """Joint attention of bf16 Q [B, S, H, D] on K/V prepared by prep_kv_bf16
    (with the same `rope`); Q RMS-normalized with `q_norm` if given.  `split`
    passes the workspace that lets a mostly idle last round of workgroups be
    split over key ranges."""
    return _fwd_prepared(load().joint_attn_fwd_bf16, "joint_attn_fwd_bf16", q, kv, rope, None,
                         softmax_scale, out, return_lse, split, q_norm, norm_eps)


def fwd_bf16(q, k, v, rope=None, softmax_scale: float = 0.0, out=None, return_lse: bool = False,
             split: bool = True, q_norm=None, k_norm=None, norm_eps: float = 0.0):
    """Joint attention on bf16 [B, S, H, D] tensors; optional Q/K RMS norm,
    RoPE from `rope` (or none): prep_kv_bf16 then fwd_bf16_prepared."""
    _check_bf16(q=q, k=k, v=v)
    if tuple(k.shape) != tuple(q.shape) or tuple(v.shape) != tuple(q.shape):
        raise ValueError("q, k, v must have the same [B, S, H, D] shape")
    kv = prep_kv_bf16(k, v, rope, k_norm, norm_eps)
    return fwd_bf16_prepared(q, kv, rope, softmax_scale, out, return_lse, split, q_norm, norm_eps)


def block_mask_shape(batch: int, seq_len: int, heads: int):
    """Shape [B, H, ceil(S / 128), ceil(S / 64)] of the block-sparse mask."""
    return (batch, heads, -(-seq_len // SPARSE_QUERY_BLOCK), -(-seq_len // SPARSE_KEY_BLOCK))


def fwd_bf16_block_sparse_prepared(q, kv, block_mask, rope=None, softmax_scale: float = 0.0,
                                   out=None, return_lse: bool = False, split: bool = True,
                                   q_norm=None, norm_eps: float = 0.0):
    """fwd_bf16_prepared restricted to the (128-query x 64-key) blocks where the
    uint8 `block_mask` [B, H, ceil(S/128), ceil(S/64)] is nonzero; query rows
    that keep no key get O = 0 and LSE = -inf."""
    want = block_mask_shape(q.shape[0], q.shape[1], q.shape[2])
    if (block_mask.dtype != torch.uint8 or tuple(block_mask.shape) != want
            or not block_mask.is_contiguous() or block_mask.device != q.device):
        raise ValueError(f"block_mask must be a contiguous uint8 {want} tensor on {q.device}")
    return _fwd_prepared(load().joint_attn_fwd_bf16_block_sparse,
                         "joint_attn_fwd_bf16_block_sparse", q, kv, rope, block_mask,
                         softmax_scale, out, return_lse, split, q_norm, norm_eps)


def fwd_bf16_block_sparse(q, k, v, block_mask, rope=None, softmax_scale: float = 0.0, out=None,
                          return_lse: bool = False, split: bool = True, q_norm=None, k_norm=None,
                          norm_eps: float = 0.0):
    """prep_kv_bf16 then fwd_bf16_block_sparse_prepared."""
    _check_bf16(q=q, k=k, v=v)
    if tuple(k.shape) != tuple(q.shape) or tuple(v.shape) != tuple(q.shape):
        raise ValueError("q, k, v must have the same [B, S, H, D] shape")
    kv = prep_kv_bf16(k, v, rope, k_norm, norm_eps)
    return fwd_bf16_block_sparse_prepared(q, kv, block_mask, rope, softmax_scale, out,
                                          return_lse, split, q_norm, norm_eps)


def _contiguous_params(batch, seq_len, heads, head_dim):
    p = Params(batch, seq_len, heads, head_dim)
    for x in "qkvo":
        setattr(p, f"{x}_sb", seq_len * heads * head_dim)
        setattr(p, f"{x}_ss", heads * head_dim)
        setattr(p, f"{x}_sh", head_dim)
    return p


def fwd_bf16_workspace_bytes(batch: int, seq_len: int, heads: int, head_dim: int) -> int:
    """Workspace of fwd_bf16 for a contiguous [B, S, H, D] call on the current
    device (0 when no split of the last round is planned)."""
    p = _contiguous_params(batch, seq_len, heads, head_dim)
    return int(load().joint_attn_fwd_bf16_workspace_bytes(ctypes.byref(p)))


def quant_rope_fp8(q, k, v, rope=None, q_norm=None, k_norm=None, norm_eps: float = 0.0):
    """Optional Q/K RMS norm, RoPE on Q/K, per-token e4m3 quantization.  Returns
    (q8, k8, v8, sq, sk, sv): uint8 codes [B, S, H, D] and fp32 scales [B, H, S]
    (powers of two for Q and K, amax/448 for V)."""
    b, s, h, d = q.shape
    dev = q.device
    q8, k8, v8 = (torch.empty((b, s, h, d), dtype=torch.uint8, device=dev) for _ in range(3))
    sq, sk, sv = (torch.empty((b, h, s), dtype=torch.float32, device=dev) for _ in range(3))
    p = _set_norm(_params(q, k, v, q, 0.0), q_norm, k_norm, norm_eps)
    st = load().joint_attn_quant_rope_fp8(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(rope),
                                          _ptr(q8), _ptr(k8), _ptr(v8), _ptr(sq), _ptr(sk),
                                          _ptr(sv), _stream(dev))
    _check(st, "joint_attn_quant_rope_fp8")
    return q8, k8, v8, sq, sk, sv


class Fp8Repair:
    """Repaired tokens of the FP8 path (from fp8_repair_plan): idx [B, H, n]
    int32, kr / vr [B, H, n_pad, D] bf16, kbias [B, H, S] fp32."""

    def __init__(self, n_rep, idx, kr, vr, kbias):
        self.n_rep, self.idx, self.kr, self.vr, self.kbias = n_rep, idx, kr, vr, kbias


def repair_count(budget: float, seq_len: int) -> int:
    """Repaired tokens per (batch, head) for a repair budget: ceil(budget * seq_len)."""
    return int(math.ceil(float(budget) * seq_len))


def fp8_repair_plan(k, v, rope, k8, v8, sk, sv, n_rep: int, k_norm=None,
                    norm_eps: float = 0.0) -> Fp8Repair:
    """Select the n_rep tokens per (batch, head) with the largest FP8 quantization
    error of their key and value, and gather their exact rotated keys and values."""
    b, s, h, d = k.shape
    dev = k.device
    n_pad = (n_rep + 31) // 32 * 32
    idx = torch.empty((b, h, n_rep), dtype=torch.int32, device=dev)
    kr = torch.empty((b, h, n_pad, d), dtype=torch.bfloat16, device=dev)
    vr = torch.empty((b, h, n_pad, d), dtype=torch.bfloat16, device=dev)
    kbias = torch.empty((b, h, s), dtype=torch.float32, device=dev)
    p = _set_norm(_params(k, k, v, k, 0.0), None, k_norm, norm_eps)
    st = load().joint_attn_fp8_repair_plan(ctypes.byref(p), _ptr(k), _ptr(v), _ptr(rope), _ptr(k8),
                                           _ptr(v8), _ptr(sk), _ptr(sv), int(n_rep),
                                           _ptr(idx) if n_rep else None, _ptr(kr), _ptr(vr),
                                           _ptr(kbias), _stream(dev))
    _check(st, "joint_attn_fp8_repair_plan")
    return Fp8Repair(n_rep, idx, kr, vr, kbias)


def _repair_c(repair):
    if repair is None or repair.n_rep <= 0:
        return None
    return Fp8RepairC(int(repair.n_rep), _ptr(repair.kbias), _ptr(repair.kr), _ptr(repair.vr))


def prep_kv_fp8(k8, v8, sk, sv, softmax_scale: float = 0.0, repair: "Fp8Repair | None" = None):
    """K/V preparation of the FP8 forward: contiguous e4m3 codes k8, v8
    [B, S, H, D] and fp32 scales sk, sv [B, H, S] (sk powers of two, as
    quant_rope_fp8 writes them) -> the prepared uint8 buffer.  The forward
    must use the same softmax_scale; `repair` removes the repaired keys."""
    b, s, h, d = k8.shape
    for t in (k8, v8):
        if t.dtype not in (torch.uint8, torch.float8_e4m3fn) or not t.is_contiguous() \
                or tuple(t.shape) != (b, s, h, d):
            raise ValueError("k8/v8 must be contiguous 1-byte [B, S, H, D] tensors")
    for t in (sk, sv):
        if t.dtype != torch.float32 or not t.is_contiguous() or tuple(t.shape) != (b, h, s):
            raise ValueError("sk/sv must be contiguous fp32 [B, H, S] tensors")
    p = Params(b, s, h, d)
    p.softmax_scale = float(softmax_scale or 0.0)
    lib = load()
    n = int(lib.joint_attn_prep_kv_fp8_bytes(ctypes.byref(p)))
    if n == 0:
        raise ValueError(f"unsupported shape {(b, s, h, d)}")
    kv8 = torch.empty(n, dtype=torch.uint8, device=k8.device)
    rc = _repair_c(repair)
    st = lib.joint_attn_prep_kv_fp8(ctypes.byref(p), _ptr(k8), _ptr(v8), _ptr(sk), _ptr(sv),
                                    ctypes.byref(rc) if rc is not None else None,
                                    _ptr(kv8), n, _stream(k8.device))
    _check(st, "joint_attn_prep_kv_fp8")
    return kv8


def fwd_fp8_prepared(q8, sq, kv8, softmax_scale: float = 0.0, out=None, return_lse: bool = False,
                     split: bool = True, repair: "Fp8Repair | None" = None):
    """FP8 forward on contiguous e4m3 q8 [B, S, H, D] with its fp32 scales sq
    [B, H, S] (powers of two; rows that meet another value come back NaN) and
    K/V prepared by prep_kv_fp8 with the same softmax_scale.  `split` as for
    fwd_bf16; `repair` from fp8_repair_plan (the one given to prep_kv_fp8)."""
    b, s, h, d = q8.shape
    if q8.dtype not in (torch.uint8, torch.float8_e4m3fn) or not q8.is_contiguous():
        raise ValueError("q8 must be a contiguous 1-byte [B, S, H, D] tensor")
    if sq.dtype != torch.float32 or not sq.is_contiguous() or tuple(sq.shape) != (b, h, s):
        raise ValueError("sq must be a contiguous fp32 [B, H, S] tensor")
    if out is None:
        out = torch.empty((b, s, h, d), dtype=torch.bfloat16, device=q8.device)
    p = Params(b, s, h, d)
    p.o_sb, p.o_ss, p.o_sh = _bshd(out, "out")
    p.softmax_scale = float(softmax_scale or 0.0)
    lse = None
    if return_lse:
        lse = torch.empty((b, h, s), dtype=torch.float32, device=q8.device)
    lib = load()
    ws_bytes = lib.joint_attn_fwd_fp8_workspace_bytes(ctypes.byref(p)) if split else 0
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=q8.device) if ws_bytes else None
    rc = _repair_c(repair)
    st = lib.joint_attn_fwd_fp8(ctypes.byref(p), _ptr(q8), _ptr(sq), _ptr(kv8), kv8.numel(),
                                ctypes.byref(rc) if rc is not None else None,
                                _ptr(out), _ptr(lse), _ptr(ws), ws_bytes, _stream(q8.device))
    _check(st, "joint_attn_fwd_fp8")
    return (out, lse) if return_lse else out


def fwd_fp8(q8, k8, v8, sq, sk, sv, softmax_scale: float = 0.0, out=None, return_lse: bool = False,
            split: bool = True, repair: "Fp8Repair | None" = None):
    """Joint attention on contiguous e4m3 codes [B, S, H, D] with fp32 scales [B, H, S]:
    prep_kv_fp8, then fwd_fp8_prepared.  sq and sk must be powers of two, as
    quant_rope_fp8 writes them (rows that meet another value come back NaN).
    `split` as for fwd_bf16; `repair` from fp8_repair_plan (None: no repair)."""
    kv8 = prep_kv_fp8(k8, v8, sk, sv, softmax_scale, repair)
    return fwd_fp8_prepared(q8, sq, kv8, softmax_scale, out, return_lse, split, repair)
