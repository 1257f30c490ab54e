"""Python binding of libjoint_attn.so (MI355X joint text+image attention).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in include/joint_attn.h, under the same
names.  PyTorch supplies device memory (outputs, workspaces) and the current
stream.  There is no fallback: if the shared library is missing or a call
fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np
import torch

__all__ = [
    "JointAttnError", "library_path", "load", "Params", "rope_table_2d",
    "fwd_bf16", "fwd_bf16_block_sparse", "prep_kv_bf16", "fwd_bf16_prepared",
    "fwd_bf16_block_sparse_prepared", "fwd_bf16_workspace_bytes", "fwd_bf16_prepared_noalloc",
    "quant_rope_fp8", "fwd_fp8", "prep_kv_fp8", "fwd_fp8_prepared", "fwd_fp8_block_sparse",
    "fwd_fp8_block_sparse_prepared",
    "Fp8Repair", "repair_count", "fp8_repair_plan",
    "SPARSE_QUERY_BLOCK", "SPARSE_KEY_BLOCK", "block_mask_shape",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
# JA_LIBRARY names another build of the same library (the host-sanitizer
# build of the C ABI tests); by default the in-tree libjoint_attn.so
_LIB_PATH = os.environ.get("JA_LIBRARY") or os.path.join(_HERE, "libjoint_attn.so")
_LIB = None

JA_OK, JA_ERR_INVALID_ARG, JA_ERR_UNSUPPORTED, JA_ERR_HIP = 0, 1, 2, 3
JA_FLAG_NO_SPLIT = 1
# block granularity of the block-sparse forwards' masks (queries x keys)
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
        ("pos", ctypes.c_void_p), ("rope_theta", ctypes.c_float),
        ("rope_table", ctypes.c_void_p), ("rope_table_bytes", ctypes.c_size_t),
        ("q_norm", ctypes.c_void_p), ("k_norm", ctypes.c_void_p),
        ("norm_eps", ctypes.c_float), ("flags", ctypes.c_uint32),
    ]


class Fp8RepairC(ctypes.Structure):
    """Mirror of ja_fp8_repair."""
    _fields_ = [("n_rep", ctypes.c_int32), ("kbias", ctypes.c_void_p),
                ("kr", ctypes.c_void_p), ("vr", ctypes.c_void_p)]


# name -> argument types (restype: ja_status unless listed in _RESTYPE)
_vp, _sz, _st = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
_pp = ctypes.POINTER(Params)
_rp = ctypes.POINTER(Fp8RepairC)
_SIGNATURES = {
    "joint_attn_rope_table_2d": [_vp, ctypes.c_int32, ctypes.c_int32, ctypes.c_float, _vp, _vp],
    "joint_attn_fwd_bf16_workspace_bytes": [_pp],
    "joint_attn_fwd_bf16": [_pp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp],
    "joint_attn_fwd_bf16_block_sparse": [_pp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp],
    "joint_attn_prep_kv_bf16_bytes": [_pp],
    "joint_attn_prep_kv_bf16": [_pp, _vp, _vp, _vp, _sz, _vp],
    "joint_attn_fwd_bf16_prepared_workspace_bytes": [_pp],
    "joint_attn_fwd_bf16_prepared": [_pp, _vp, _vp, _sz, _vp, _vp, _vp, _sz, _vp],
    "joint_attn_fwd_bf16_block_sparse_prepared": [_pp, _vp, _vp, _sz, _vp, _vp, _vp, _vp, _sz,
                                                  _vp],
    "joint_attn_fwd_bf16_prepared_noalloc": [_pp, _vp, _vp, _sz, _vp, _vp, _vp],
    "joint_attn_quant_rope_fp8_workspace_bytes": [_pp],
    "joint_attn_quant_rope_fp8": [_pp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz,
                                  _vp],
    "joint_attn_fwd_fp8_workspace_bytes": [_pp],
    "joint_attn_fwd_fp8": [_pp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp],
    "joint_attn_fwd_fp8_block_sparse": [_pp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                        _sz, _vp],
    "joint_attn_fwd_fp8_block_sparse_prepared": [_pp, _vp, _vp, _vp, _sz, _vp, _vp, _vp, _vp,
                                                 _sz, _vp],
    "joint_attn_fp8_repair_count": [ctypes.c_double, ctypes.c_int32],
    "joint_attn_fp8_repair_plan_workspace_bytes": [_pp],
    "joint_attn_fp8_repair_plan": [_pp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_int32, _vp, _vp,
                                   _vp, _vp, _vp, _sz, _vp],
    "joint_attn_prep_kv_fp8_bytes": [_pp],
    "joint_attn_prep_kv_fp8": [_pp, _vp, _vp, _vp, _vp, _rp, _vp, _sz, _vp],
    "joint_attn_fwd_fp8_prepared_workspace_bytes": [_pp],
    "joint_attn_fwd_fp8_prepared": [_pp, _vp, _vp, _vp, _sz, _rp, _vp, _vp, _vp, _sz, _vp],
    "joint_attn_status_string": [_st],
    "joint_attn_last_error": [],
}
_RESTYPE = {"joint_attn_status_string": ctypes.c_char_p,
            "joint_attn_last_error": ctypes.c_char_p,
            "joint_attn_fp8_repair_count": ctypes.c_int32}


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
    for name, args in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = _RESTYPE.get(name, _sz if name.endswith("_bytes") else _st)
    _LIB = lib
    return lib


def _check(status: int, fn: str) -> None:
    if status != JA_OK:
        lib = load()
        msg = lib.joint_attn_status_string(status).decode()
        raise JointAttnError(status, f"{fn}: {msg}: {lib.joint_attn_last_error().decode()}")


def _call(name: str, *args) -> None:
    _check(getattr(load(), name)(*args), name)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _scratch(nbytes: int, device):
    """A uint8 device tensor of nbytes (None for 0): workspaces come from
    torch's stream-ordered allocator."""
    return torch.empty(int(nbytes), dtype=torch.uint8, device=device) if nbytes else None


def _need_device(t, name, device):
    if not t.is_cuda or (device is not None and t.device != torch.device(device)):
        raise ValueError(f"{name} must be a tensor on {device}")


def _bshd(t: torch.Tensor, name: str, dtype=torch.bfloat16, shape=None, device=None):
    """Strides (sb, ss, sh) of a [B, S, H, D] tensor with unit D stride."""
    if t.dim() != 4:
        raise ValueError(f"{name} must be 4-D [B, S, H, D], got {tuple(t.shape)}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} shape {tuple(t.shape)} != {tuple(shape)}")
    if t.stride(3) != 1:
        raise ValueError(f"{name} must have a unit stride along D")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}")
    _need_device(t, name, device if device is not None else t.device)
    return t.stride(0), t.stride(1), t.stride(2)


def _contiguous_1byte(t, name, shape, device):
    if t.dtype not in (torch.uint8, torch.float8_e4m3fn) or not t.is_contiguous() \
            or tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must be a contiguous 1-byte {tuple(shape)} tensor")
    _need_device(t, name, device)


def _contiguous_f32(t, name, shape, device, dtype=torch.float32):
    if t.dtype != dtype or not t.is_contiguous() or tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must be a contiguous {dtype} {tuple(shape)} tensor")
    _need_device(t, name, device)


class _Call:
    """ja_params of one call plus the tensors it points to (kept alive until
    the call has been enqueued)."""

    def __init__(self, shape, device, softmax_scale=0.0, split=True):
        b, s, h, d = shape
        self.shape, self.device = tuple(shape), torch.device(device)
        self.p = Params(b, s, h, d)
        self.p.softmax_scale = float(softmax_scale or 0.0)
        self.p.flags = 0 if split else JA_FLAG_NO_SPLIT
        self.keep = []

    def strides(self, which, t, name, dtype=torch.bfloat16):
        sb, ss, sh = _bshd(t, name, dtype, self.shape, self.device)
        setattr(self.p, f"{which}_sb", sb)
        setattr(self.p, f"{which}_ss", ss)
        setattr(self.p, f"{which}_sh", sh)

    def rope(self, pos=None, theta=10000.0, rope=None):
        """RoPE from int32 positions [S, 2] (device tensor or array) and/or a
        prebuilt table from rope_table_2d (fp64 [S, D/2, 2] on the device)."""
        s, d = self.shape[1], self.shape[3]
        if pos is not None:
            if not torch.is_tensor(pos):
                pos = torch.from_numpy(np.ascontiguousarray(pos, dtype=np.int32))
            pos = pos.to(self.device)
            if pos.dtype != torch.int32 or tuple(pos.shape) != (s, 2) or not pos.is_contiguous():
                raise ValueError(f"pos must be a contiguous int32 [{s}, 2] tensor")
            self.keep.append(pos)
            self.p.pos = pos.data_ptr()
        self.p.rope_theta = float(theta)
        if rope is not None:
            _contiguous_f32(rope, "rope", (s, d // 2, 2), self.device, torch.float64)
            self.p.rope_table = rope.data_ptr()
            self.p.rope_table_bytes = rope.numel() * 8
        return self

    def norm(self, q_norm=None, k_norm=None, norm_eps=0.0):
        """Optional query/key RMS-norm weights: fp32 contiguous [head_dim]
        device tensors (None = that tensor is not normalized); norm_eps 0 = 1e-6."""
        d = self.shape[3]
        for t, n in ((q_norm, "q_norm"), (k_norm, "k_norm")):
            if t is not None:
                _contiguous_f32(t, n, (d,), self.device)
        self.p.q_norm = None if q_norm is None else q_norm.data_ptr()
        self.p.k_norm = None if k_norm is None else k_norm.data_ptr()
        self.p.norm_eps = float(norm_eps)
        return self

    def ref(self):
        return ctypes.byref(self.p)

    def query(self, name) -> int:
        return int(getattr(load(), name)(self.ref()))

    def stream(self):
        return _stream(self.device)


def rope_table_2d(pos: torch.Tensor, head_dim: int, theta: float = 10000.0) -> torch.Tensor:
    """(cos, sin) table [S, head_dim/2, 2] fp64 of 2D-axial RoPE for int32 pos [S, 2]."""
    if pos.dtype != torch.int32 or pos.dim() != 2 or pos.shape[1] != 2 or not pos.is_contiguous() \
            or not pos.is_cuda:
        raise ValueError("pos must be a contiguous int32 [S, 2] device tensor")
    table = torch.empty((pos.shape[0], head_dim // 2, 2), dtype=torch.float64, device=pos.device)
    _call("joint_attn_rope_table_2d", _ptr(pos), pos.shape[0], head_dim, float(theta),
          _ptr(table), _stream(pos.device))
    return table


def _out_lse(c: _Call, out, return_lse):
    b, s, h, d = c.shape
    if out is None:
        out = torch.empty((b, s, h, d), dtype=torch.bfloat16, device=c.device)
    c.strides("o", out, "out")
    lse = torch.empty((b, h, s), dtype=torch.float32, device=c.device) if return_lse else None
    return out, lse


def block_mask_shape(batch: int, seq_len: int, heads: int):
    """Shape [B, H, ceil(S / 128), ceil(S / 64)] of a block-sparse mask."""
    return (batch, heads, -(-seq_len // SPARSE_QUERY_BLOCK), -(-seq_len // SPARSE_KEY_BLOCK))


def _check_mask(c: _Call, block_mask):
    want = block_mask_shape(c.shape[0], c.shape[1], c.shape[2])
    if (block_mask.dtype != torch.uint8 or tuple(block_mask.shape) != want
            or not block_mask.is_contiguous() or block_mask.device != c.device):
        raise ValueError(f"block_mask must be a contiguous uint8 {want} tensor on {c.device}")


# ---- BF16 path ----

def _bf16_call(q, k, v, pos, theta, rope, softmax_scale, split, q_norm, k_norm, norm_eps):
    c = _Call(q.shape, q.device, softmax_scale, split)
    c.strides("q", q, "q")
    c.strides("k", k, "k")
    c.strides("v", v, "v")
    return c.rope(pos, theta, rope).norm(q_norm, k_norm, norm_eps)


def fwd_bf16(q, k, v, pos=None, theta: float = 10000.0, rope=None, softmax_scale: float = 0.0,
             out=None, return_lse: bool = False, split: bool = True, q_norm=None, k_norm=None,
             norm_eps: float = 0.0):
    """Joint attention of bf16 Q, K, V [B, S, H, D] (joint_attn_fwd_bf16).

    RoPE at int32 grid positions `pos` [S, 2] with base `theta` (or the table
    `rope` from rope_table_2d); optional Q/K RMS norm weights; `split=False`
    sets JA_FLAG_NO_SPLIT.  Returns out (and the LSE [B, H, S] with return_lse)."""
    c = _bf16_call(q, k, v, pos, theta, rope, softmax_scale, split, q_norm, k_norm, norm_eps)
    out, lse = _out_lse(c, out, return_lse)
    n = c.query("joint_attn_fwd_bf16_workspace_bytes")
    ws = _scratch(n, c.device)
    _call("joint_attn_fwd_bf16", c.ref(), _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse),
          _ptr(ws), n, c.stream())
    return (out, lse) if return_lse else out


def fwd_bf16_block_sparse(q, k, v, block_mask, pos=None, theta: float = 10000.0, rope=None,
                          softmax_scale: float = 0.0, out=None, return_lse: bool = False,
                          split: bool = True, q_norm=None, k_norm=None, norm_eps: float = 0.0):
    """fwd_bf16 restricted to the (128-query x 64-key) blocks where the uint8
    `block_mask` [B, H, ceil(S/128), ceil(S/64)] is nonzero; query rows that
    keep no key get O = 0 and LSE = -inf (joint_attn_fwd_bf16_block_sparse)."""
    c = _bf16_call(q, k, v, pos, theta, rope, softmax_scale, split, q_norm, k_norm, norm_eps)
    _check_mask(c, block_mask)
    out, lse = _out_lse(c, out, return_lse)
    n = c.query("joint_attn_fwd_bf16_workspace_bytes")
    ws = _scratch(n, c.device)
    _call("joint_attn_fwd_bf16_block_sparse", c.ref(), _ptr(q), _ptr(k), _ptr(v),
          _ptr(block_mask), _ptr(out), _ptr(lse), _ptr(ws), n, c.stream())
    return (out, lse) if return_lse else out


def fwd_bf16_workspace_bytes(batch: int, seq_len: int, heads: int, head_dim: int,
                             rope: bool = True, split: bool = True) -> int:
    """Workspace of joint_attn_fwd_bf16 for contiguous [B, S, H, D] tensors."""
    c = _Call((batch, seq_len, heads, head_dim), "cpu", 0.0, split)
    for x in "qkvo":
        setattr(c.p, f"{x}_sb", seq_len * heads * head_dim)
        setattr(c.p, f"{x}_ss", heads * head_dim)
        setattr(c.p, f"{x}_sh", head_dim)
    if rope:
        c.p.pos = 16      # any aligned non-NULL pointer: only its presence matters here
    return c.query("joint_attn_fwd_bf16_workspace_bytes")


def prep_kv_bf16(k, v, pos=None, theta: float = 10000.0, rope=None, k_norm=None,
                 norm_eps: float = 0.0):
    """Prepared K/V buffer of the bf16 forward (uint8 device tensor;
    joint_attn_prep_kv_bf16): K RMS-normalized (k_norm) and rotated, V
    transposed, plus the RoPE table when only `pos` is given."""
    c = _Call(k.shape, k.device)
    c.strides("k", k, "k")
    c.strides("v", v, "v")
    c.rope(pos, theta, rope).norm(None, k_norm, norm_eps)
    n = c.query("joint_attn_prep_kv_bf16_bytes")
    if n == 0:
        raise JointAttnError(JA_ERR_UNSUPPORTED, "joint_attn_prep_kv_bf16: unsupported shape")
    kv = torch.empty(n, dtype=torch.uint8, device=k.device)
    _call("joint_attn_prep_kv_bf16", c.ref(), _ptr(k), _ptr(v), _ptr(kv), n, c.stream())
    return kv


def _prepared_bf16(name, q, kv, mask, pos, theta, rope, softmax_scale, out, return_lse, split,
                   q_norm, norm_eps):
    c = _Call(q.shape, q.device, softmax_scale, split)
    c.strides("q", q, "q")
    c.rope(pos, theta, rope).norm(q_norm, None, norm_eps)
    if kv.dtype != torch.uint8 or kv.dim() != 1 or kv.device != c.device:
        raise ValueError("kv must be the uint8 buffer from prep_kv_bf16 on q's device")
    if mask is not None:
        _check_mask(c, mask)
    out, lse = _out_lse(c, out, return_lse)
    n = c.query("joint_attn_fwd_bf16_prepared_workspace_bytes")
    ws = _scratch(n, c.device)
    args = [c.ref(), _ptr(q), _ptr(kv), kv.numel()] + ([_ptr(mask)] if mask is not None else [])
    _call(name, *args, _ptr(out), _ptr(lse), _ptr(ws), n, c.stream())
    return (out, lse) if return_lse else out


def fwd_bf16_prepared(q, kv, pos=None, theta: float = 10000.0, rope=None,
                      softmax_scale: float = 0.0, out=None, return_lse: bool = False,
                      split: bool = True, q_norm=None, norm_eps: float = 0.0):
    """Attention of bf16 Q on K/V from prep_kv_bf16 (prepared with the same
    pos / rope): joint_attn_fwd_bf16_prepared."""
    return _prepared_bf16("joint_attn_fwd_bf16_prepared", q, kv, None, pos, theta, rope,
                          softmax_scale, out, return_lse, split, q_norm, norm_eps)


def fwd_bf16_prepared_noalloc(q, kv, pos=None, theta: float = 10000.0, rope=None,
                              softmax_scale: float = 0.0, out=None, return_lse: bool = False,
                              split: bool = True, q_norm=None, norm_eps: float = 0.0):
    """fwd_bf16_prepared with the library's static scratch instead of a
    workspace (joint_attn_fwd_bf16_prepared_noalloc): the call allocates
    nothing (pass `out`, and `pos`/`rope` already on the device, to allocate
    nothing here either)."""
    c = _Call(q.shape, q.device, softmax_scale, split)
    c.strides("q", q, "q")
    c.rope(pos, theta, rope).norm(q_norm, None, norm_eps)
    if kv.dtype != torch.uint8 or kv.dim() != 1 or kv.device != c.device:
        raise ValueError("kv must be the uint8 buffer from prep_kv_bf16 on q's device")
    out, lse = _out_lse(c, out, return_lse)
    _call("joint_attn_fwd_bf16_prepared_noalloc", c.ref(), _ptr(q), _ptr(kv), kv.numel(),
          _ptr(out), _ptr(lse), c.stream())
    return (out, lse) if return_lse else out


def fwd_bf16_block_sparse_prepared(q, kv, block_mask, pos=None, theta: float = 10000.0,
                                   rope=None, softmax_scale: float = 0.0, out=None,
                                   return_lse: bool = False, split: bool = True, q_norm=None,
                                   norm_eps: float = 0.0):
    """fwd_bf16_prepared restricted to the blocks of `block_mask`
    (joint_attn_fwd_bf16_block_sparse_prepared)."""
    return _prepared_bf16("joint_attn_fwd_bf16_block_sparse_prepared", q, kv, block_mask, pos,
                          theta, rope, softmax_scale, out, return_lse, split, q_norm, norm_eps)


# ---- FP8 path ----

def quant_rope_fp8(q, k, v, pos=None, theta: float = 10000.0, rope=None, q_norm=None,
                   k_norm=None, norm_eps: float = 0.0):
    """Optional Q/K RMS norm, RoPE on Q/K, per-token e4m3 quantization
    (joint_attn_quant_rope_fp8).  Returns (q8, k8, v8, sq, sk, sv): uint8
    codes [B, S, H, D] and fp32 scales [B, H, S] (powers of two for Q and K,
    amax/448 for V)."""
    b, s, h, d = q.shape
    c = _bf16_call(q, k, v, pos, theta, rope, 0.0, True, q_norm, k_norm, norm_eps)
    dev = c.device
    q8, k8, v8 = (torch.empty((b, s, h, d), dtype=torch.uint8, device=dev) for _ in range(3))
    sq, sk, sv = (torch.empty((b, h, s), dtype=torch.float32, device=dev) for _ in range(3))
    n = c.query("joint_attn_quant_rope_fp8_workspace_bytes")
    ws = _scratch(n, dev)
    _call("joint_attn_quant_rope_fp8", c.ref(), _ptr(q), _ptr(k), _ptr(v), _ptr(q8), _ptr(k8),
          _ptr(v8), _ptr(sq), _ptr(sk), _ptr(sv), _ptr(ws), n, c.stream())
    return q8, k8, v8, sq, sk, sv


def _fp8_call(shape, device, softmax_scale, split, codes, scales):
    b, s, h, d = shape
    c = _Call(shape, device, softmax_scale, split)
    for t, n in codes:
        _contiguous_1byte(t, n, (b, s, h, d), c.device)
    for t, n in scales:
        _contiguous_f32(t, n, (b, h, s), c.device)
    return c


def fwd_fp8(q8, k8, v8, sq, sk, sv, softmax_scale: float = 0.0, out=None,
            return_lse: bool = False, split: bool = True):
    """Joint attention on contiguous e4m3 codes [B, S, H, D] with fp32 scales
    [B, H, S] (joint_attn_fwd_fp8).  sq and sk must be powers of two, as
    quant_rope_fp8 writes them (rows that meet another value come back NaN)."""
    c = _fp8_call(q8.shape, q8.device, softmax_scale, split,
                  ((q8, "q8"), (k8, "k8"), (v8, "v8")), ((sq, "sq"), (sk, "sk"), (sv, "sv")))
    out, lse = _out_lse(c, out, return_lse)
    n = c.query("joint_attn_fwd_fp8_workspace_bytes")
    ws = _scratch(n, c.device)
    _call("joint_attn_fwd_fp8", c.ref(), _ptr(q8), _ptr(k8), _ptr(v8), _ptr(sq), _ptr(sk),
          _ptr(sv), _ptr(out), _ptr(lse), _ptr(ws), n, c.stream())
    return (out, lse) if return_lse else out


def fwd_fp8_block_sparse(q8, k8, v8, sq, sk, sv, block_mask, softmax_scale: float = 0.0,
                         out=None, return_lse: bool = False, split: bool = True):
    """fwd_fp8 restricted to the (128-query x 64-key) blocks where the uint8
    `block_mask` [B, H, ceil(S/128), ceil(S/64)] is nonzero; query rows that
    keep no key get O = 0 and LSE = -inf (joint_attn_fwd_fp8_block_sparse)."""
    c = _fp8_call(q8.shape, q8.device, softmax_scale, split,
                  ((q8, "q8"), (k8, "k8"), (v8, "v8")), ((sq, "sq"), (sk, "sk"), (sv, "sv")))
    _check_mask(c, block_mask)
    out, lse = _out_lse(c, out, return_lse)
    n = c.query("joint_attn_fwd_fp8_workspace_bytes")
    ws = _scratch(n, c.device)
    _call("joint_attn_fwd_fp8_block_sparse", c.ref(), _ptr(q8), _ptr(k8), _ptr(v8), _ptr(sq),
          _ptr(sk), _ptr(sv), _ptr(block_mask), _ptr(out), _ptr(lse), _ptr(ws), n, c.stream())
    return (out, lse) if return_lse else out


def fwd_fp8_block_sparse_prepared(q8, sq, kv8, block_mask, softmax_scale: float = 0.0, out=None,
                                  return_lse: bool = False, split: bool = True):
    """fwd_fp8_block_sparse on K/V from prep_kv_fp8 (prepared with the same
    softmax_scale): joint_attn_fwd_fp8_block_sparse_prepared."""
    c = _fp8_call(q8.shape, q8.device, softmax_scale, split, ((q8, "q8"),), ((sq, "sq"),))
    _check_mask(c, block_mask)
    if kv8.dtype != torch.uint8 or kv8.dim() != 1 or kv8.device != c.device:
        raise ValueError("kv8 must be the uint8 buffer from prep_kv_fp8 on q8's device")
    out, lse = _out_lse(c, out, return_lse)
    n = c.query("joint_attn_fwd_fp8_prepared_workspace_bytes")
    ws = _scratch(n, c.device)
    _call("joint_attn_fwd_fp8_block_sparse_prepared", c.ref(), _ptr(q8), _ptr(sq), _ptr(kv8),
          kv8.numel(), _ptr(block_mask), _ptr(out), _ptr(lse), _ptr(ws), n, c.stream())
    return (out, lse) if return_lse else out


class Fp8Repair:
    """Repaired tokens of the FP8 path (from fp8_repair_plan): idx [B, H, n]
    int32, kr / vr [B, H, n_pad, D] bf16, kbias [B, H, S] fp32."""

    def __init__(self, n_rep, idx, kr, vr, kbias):
        self.n_rep, self.idx, self.kr, self.vr, self.kbias = n_rep, idx, kr, vr, kbias


def repair_count(budget: float, seq_len: int) -> int:
    """Repaired tokens per (batch, head) for a repair budget
    (joint_attn_fp8_repair_count)."""
    n = int(load().joint_attn_fp8_repair_count(float(budget), int(seq_len)))
    if n < 0:
        raise JointAttnError(JA_ERR_INVALID_ARG, "joint_attn_fp8_repair_count: "
                             + load().joint_attn_last_error().decode())
    return n


def fp8_repair_plan(k, v, k8, v8, sk, sv, n_rep: int, pos=None, theta: float = 10000.0,
                    rope=None, k_norm=None, norm_eps: float = 0.0) -> Fp8Repair:
    """Select the n_rep tokens per (batch, head) with the largest FP8 quantization
    error of their key and value, and gather their exact rotated keys and values
    (joint_attn_fp8_repair_plan)."""
    b, s, h, d = k.shape
    c = _Call(k.shape, k.device)
    c.strides("k", k, "k")
    c.strides("v", v, "v")
    c.rope(pos, theta, rope).norm(None, k_norm, norm_eps)
    dev = c.device
    for t, n in ((k8, "k8"), (v8, "v8")):
        _contiguous_1byte(t, n, (b, s, h, d), dev)
    for t, n in ((sk, "sk"), (sv, "sv")):
        _contiguous_f32(t, n, (b, h, s), dev)
    n_pad = (n_rep + 31) // 32 * 32
    idx = torch.empty((b, h, n_rep), dtype=torch.int32, device=dev)
    kr = torch.empty((b, h, n_pad, d), dtype=torch.bfloat16, device=dev)
    vr = torch.empty((b, h, n_pad, d), dtype=torch.bfloat16, device=dev)
    kbias = torch.empty((b, h, s), dtype=torch.float32, device=dev)
    n = c.query("joint_attn_fp8_repair_plan_workspace_bytes")
    ws = _scratch(n, dev)
    _call("joint_attn_fp8_repair_plan", c.ref(), _ptr(k), _ptr(v), _ptr(k8), _ptr(v8), _ptr(sk),
          _ptr(sv), int(n_rep), _ptr(idx) if n_rep else None, _ptr(kr), _ptr(vr), _ptr(kbias),
          _ptr(ws), n, c.stream())
    return Fp8Repair(n_rep, idx, kr, vr, kbias)


def _repair_c(repair):
    if repair is None or repair.n_rep <= 0:
        return None
    return Fp8RepairC(int(repair.n_rep), _ptr(repair.kbias), _ptr(repair.kr), _ptr(repair.vr))


def prep_kv_fp8(k8, v8, sk, sv, softmax_scale: float = 0.0, repair: "Fp8Repair | None" = None):
    """K/V preparation of the FP8 forward (joint_attn_prep_kv_fp8): contiguous
    e4m3 codes k8, v8 [B, S, H, D] and fp32 scales sk, sv [B, H, S] -> the
    prepared uint8 buffer.  The forward must use the same softmax_scale;
    `repair` removes the repaired keys."""
    c = _fp8_call(k8.shape, k8.device, softmax_scale, True, ((k8, "k8"), (v8, "v8")),
                  ((sk, "sk"), (sv, "sv")))
    n = c.query("joint_attn_prep_kv_fp8_bytes")
    if n == 0:
        raise JointAttnError(JA_ERR_UNSUPPORTED, f"unsupported shape {tuple(k8.shape)}")
    kv8 = torch.empty(n, dtype=torch.uint8, device=c.device)
    rc = _repair_c(repair)
    _call("joint_attn_prep_kv_fp8", c.ref(), _ptr(k8), _ptr(v8), _ptr(sk), _ptr(sv),
          ctypes.byref(rc) if rc is not None else None, _ptr(kv8), n, c.stream())
    return kv8


def fwd_fp8_prepared(q8, sq, kv8, softmax_scale: float = 0.0, out=None, return_lse: bool = False,
                     split: bool = True, repair: "Fp8Repair | None" = None):
    """FP8 forward on contiguous e4m3 q8 [B, S, H, D] with its fp32 scales sq
    [B, H, S] and K/V prepared by prep_kv_fp8 with the same softmax_scale
    (joint_attn_fwd_fp8_prepared); `repair` from fp8_repair_plan (the one
    given to prep_kv_fp8)."""
    c = _fp8_call(q8.shape, q8.device, softmax_scale, split, ((q8, "q8"),), ((sq, "sq"),))
    if kv8.dtype != torch.uint8 or kv8.dim() != 1 or kv8.device != c.device:
        raise ValueError("kv8 must be the uint8 buffer from prep_kv_fp8 on q8's device")
    out, lse = _out_lse(c, out, return_lse)
    n = c.query("joint_attn_fwd_fp8_prepared_workspace_bytes")
    ws = _scratch(n, c.device)
    rc = _repair_c(repair)
    _call("joint_attn_fwd_fp8_prepared", c.ref(), _ptr(q8), _ptr(sq), _ptr(kv8), kv8.numel(),
          ctypes.byref(rc) if rc is not None else None, _ptr(out), _ptr(lse), _ptr(ws), n,
          c.stream())
    return (out, lse) if return_lse else out
