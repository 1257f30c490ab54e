"""C ABI checks that need no GPU: the library loads, exports every function
that include/joint_attn.h declares, and rejects invalid calls on the host
before anything is enqueued (the pointers below are never dereferenced)."""
import ctypes
import os
import re

import pytest

import joint_attention_attn_amd as ja

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "joint_attn.h")
FAKE = 0x10000  # 16-byte aligned stand-in address; validation fails before use


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(ja.library_path()):
        pytest.fail("libjoint_attn.so is not built (run __graft_entry__.build())")
    return ja.load()


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(joint_attn_\w+)\s*\(", text)))


def test_every_declared_symbol_is_exported(lib):
    names = _declared()
    assert {"joint_attn_fwd_bf16", "joint_attn_fwd_fp8", "joint_attn_quant_rope_fp8",
            "joint_attn_rope_table_2d", "joint_attn_status_string"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(lib):
    for code in range(4):
        assert lib.joint_attn_status_string(code).startswith(b"JA_")
    assert lib.joint_attn_status_string(99) == b"unknown ja_status"


def _p(b=1, s=80, h=2, d=64):
    p = ja.Params(b, s, h, d)
    for x in "qkvo":
        setattr(p, f"{x}_sb", s * h * d)
        setattr(p, f"{x}_ss", h * d)
        setattr(p, f"{x}_sh", d)
    return p


KV_BYTES = 1 << 30   # stand-in size of the prepared K/V buffer


def _fwd(lib, p, q=FAKE, kv=FAKE + 0x1000, o=FAKE + 0x3000, rope=None, lse=None,
         ws=None, ws_bytes=0, kv_bytes=KV_BYTES):
    vp = ctypes.c_void_p
    return lib.joint_attn_fwd_bf16(ctypes.byref(p) if p is not None else None, vp(q), vp(kv),
                                   kv_bytes, vp(rope), vp(o), vp(lse), vp(ws), ws_bytes, None)


@pytest.mark.parametrize("mutate,expect", [
    (lambda p: setattr(p, "batch", 0), ja.JA_ERR_INVALID_ARG),
    (lambda p: setattr(p, "seq_len", 0), ja.JA_ERR_INVALID_ARG),
    (lambda p: setattr(p, "heads", -1), ja.JA_ERR_INVALID_ARG),
    (lambda p: setattr(p, "head_dim", 96), ja.JA_ERR_UNSUPPORTED),
    (lambda p: setattr(p, "head_dim", 256), ja.JA_ERR_UNSUPPORTED),
    (lambda p: setattr(p, "q_ss", 100), ja.JA_ERR_INVALID_ARG),
    (lambda p: setattr(p, "k_sh", 4), ja.JA_ERR_INVALID_ARG),
    (lambda p: setattr(p, "o_sb", -8), ja.JA_ERR_INVALID_ARG),
    (lambda p: setattr(p, "softmax_scale", float("nan")), ja.JA_ERR_INVALID_ARG),
    (lambda p: setattr(p, "softmax_scale", -1.0), ja.JA_ERR_INVALID_ARG),
    (lambda p: setattr(p, "heads", 70000), ja.JA_ERR_UNSUPPORTED),
])
def test_fwd_bf16_rejects_bad_params(lib, mutate, expect):
    p = _p()
    mutate(p)
    assert _fwd(lib, p) == expect


def test_fwd_bf16_rejects_bad_pointers(lib):
    assert _fwd(lib, None) == ja.JA_ERR_INVALID_ARG
    assert _fwd(lib, _p(), q=0) == ja.JA_ERR_INVALID_ARG
    assert _fwd(lib, _p(), o=0) == ja.JA_ERR_INVALID_ARG
    assert _fwd(lib, _p(), kv=FAKE + 2) == ja.JA_ERR_INVALID_ARG        # misaligned
    assert _fwd(lib, _p(), kv=0) == ja.JA_ERR_INVALID_ARG
    assert _fwd(lib, _p(), kv_bytes=1024) == ja.JA_ERR_INVALID_ARG      # too small
    assert _fwd(lib, _p(), rope=FAKE + 8) == ja.JA_ERR_INVALID_ARG      # misaligned table
    assert _fwd(lib, _p(), lse=FAKE + 2) == ja.JA_ERR_INVALID_ARG
    assert _fwd(lib, _p(), o=FAKE) == ja.JA_ERR_INVALID_ARG             # o aliases q
    assert _fwd(lib, _p(), ws=FAKE + 0x4008, ws_bytes=64) == ja.JA_ERR_INVALID_ARG  # misaligned


def test_workspace_bytes_of_invalid_params_is_zero(lib):
    assert lib.joint_attn_fwd_bf16_workspace_bytes(None) == 0
    bad = _p()
    bad.head_dim = 96
    assert lib.joint_attn_fwd_bf16_workspace_bytes(ctypes.byref(bad)) == 0


def test_rope_table_validation(lib):
    vp = ctypes.c_void_p
    f = lib.joint_attn_rope_table_2d
    assert f(vp(0), 10, 64, 10000.0, vp(FAKE), None) == ja.JA_ERR_INVALID_ARG
    assert f(vp(FAKE), 0, 64, 10000.0, vp(FAKE), None) == ja.JA_ERR_INVALID_ARG
    assert f(vp(FAKE), 10, 64, 0.0, vp(FAKE), None) == ja.JA_ERR_INVALID_ARG
    assert f(vp(FAKE), 10, 64, float("inf"), vp(FAKE), None) == ja.JA_ERR_INVALID_ARG
    assert f(vp(FAKE), 10, 48, 10000.0, vp(FAKE), None) == ja.JA_ERR_UNSUPPORTED
    assert f(vp(FAKE), 10, 64, 10000.0, vp(FAKE + 4), None) == ja.JA_ERR_INVALID_ARG


def test_quant_and_fp8_validation(lib):
    vp = ctypes.c_void_p
    p = _p()
    ptrs = [vp(FAKE + 0x1000 * i) for i in range(10)]
    bad = _p()
    bad.head_dim = 32
    assert lib.joint_attn_quant_rope_fp8(ctypes.byref(bad), *ptrs[:3], None, *ptrs[3:6],
                                         *ptrs[6:9], None) == ja.JA_ERR_UNSUPPORTED
    assert lib.joint_attn_quant_rope_fp8(ctypes.byref(p), vp(0), *ptrs[1:3], None, *ptrs[3:6],
                                         *ptrs[6:9], None) == ja.JA_ERR_INVALID_ARG


def _fwd8(lib, p, q8=FAKE, sq=FAKE + 0x1000, kv8=FAKE + 0x2000, kv8_bytes=KV_BYTES, rep=None,
          o=FAKE + 0x3000, lse=None, ws=None, ws_bytes=0):
    vp = ctypes.c_void_p
    return lib.joint_attn_fwd_fp8(ctypes.byref(p), vp(q8), vp(sq), vp(kv8), kv8_bytes,
                                  ctypes.byref(rep) if rep is not None else None, vp(o),
                                  vp(lse) if lse else None, vp(ws) if ws else None, ws_bytes, None)


def _prep8(lib, p, k8=FAKE, v8=FAKE + 0x1000, sk=FAKE + 0x2000, sv=FAKE + 0x3000, rep=None,
           kv8=FAKE + 0x4000, kv8_bytes=KV_BYTES):
    vp = ctypes.c_void_p
    return lib.joint_attn_prep_kv_fp8(ctypes.byref(p), vp(k8), vp(v8), vp(sk), vp(sv),
                                      ctypes.byref(rep) if rep is not None else None, vp(kv8),
                                      kv8_bytes, None)


def test_fp8_prep_and_forward_validation(lib):
    p = _p()
    bad = _p()
    bad.head_dim = 32
    # prepared size: K and V^T of S_pad = 128 keys, one 1 KB block per 64-key tile
    n = lib.joint_attn_prep_kv_fp8_bytes(ctypes.byref(p))
    assert n == 1 * 2 * (2 * 128 * 64 + 2 * 1024)
    assert lib.joint_attn_prep_kv_fp8_bytes(ctypes.byref(bad)) == 0
    assert _prep8(lib, bad) == ja.JA_ERR_UNSUPPORTED
    assert _prep8(lib, p, k8=0) == ja.JA_ERR_INVALID_ARG
    assert _prep8(lib, p, sk=FAKE + 0x2002) == ja.JA_ERR_INVALID_ARG
    assert _prep8(lib, p, kv8=FAKE + 0x4004) == ja.JA_ERR_INVALID_ARG
    assert _prep8(lib, p, kv8_bytes=n - 1) == ja.JA_ERR_INVALID_ARG
    assert _prep8(lib, p, rep=ja.Fp8RepairC(5, None, FAKE, FAKE)) == ja.JA_ERR_INVALID_ARG
    assert _prep8(lib, p, rep=ja.Fp8RepairC(81, FAKE, FAKE, FAKE)) == ja.JA_ERR_INVALID_ARG
    assert _prep8(lib, p, rep=ja.Fp8RepairC(-1, FAKE, FAKE, FAKE)) == ja.JA_ERR_INVALID_ARG

    assert _fwd8(lib, bad) == ja.JA_ERR_UNSUPPORTED
    assert _fwd8(lib, p, q8=FAKE + 4) == ja.JA_ERR_INVALID_ARG
    assert _fwd8(lib, p, sq=FAKE + 0x1002) == ja.JA_ERR_INVALID_ARG
    assert _fwd8(lib, p, o=0) == ja.JA_ERR_INVALID_ARG
    assert _fwd8(lib, p, o=FAKE) == ja.JA_ERR_INVALID_ARG            # aliases q8
    assert _fwd8(lib, p, kv8_bytes=n - 1) == ja.JA_ERR_INVALID_ARG
    assert _fwd8(lib, p, ws=FAKE + 0x9008, ws_bytes=64) == ja.JA_ERR_INVALID_ARG
    assert _fwd8(lib, p, rep=ja.Fp8RepairC(5, FAKE, None, FAKE)) == ja.JA_ERR_INVALID_ARG
    assert _fwd8(lib, p, rep=ja.Fp8RepairC(81, FAKE, FAKE, FAKE)) == ja.JA_ERR_INVALID_ARG


def test_repair_plan_validation(lib):
    vp = ctypes.c_void_p
    p = _p()
    ptrs = [vp(FAKE + 0x1000 * i) for i in range(12)]
    f = lib.joint_attn_fp8_repair_plan
    assert f(ctypes.byref(p), *ptrs[:2], None, *ptrs[2:6], 81, *ptrs[6:10], None) == ja.JA_ERR_INVALID_ARG
    assert f(ctypes.byref(p), *ptrs[:2], None, *ptrs[2:6], -1, *ptrs[6:10], None) == ja.JA_ERR_INVALID_ARG
    assert f(ctypes.byref(p), *ptrs[:2], None, *ptrs[2:6], 4, None, *ptrs[7:10], None) == ja.JA_ERR_INVALID_ARG
    long = _p(s=40000)
    assert f(ctypes.byref(long), *ptrs[:2], None, *ptrs[2:6], 4, *ptrs[6:10], None) == ja.JA_ERR_UNSUPPORTED
    bad = _p()
    bad.head_dim = 96
    assert f(ctypes.byref(bad), *ptrs[:2], None, *ptrs[2:6], 4, *ptrs[6:10], None) == ja.JA_ERR_UNSUPPORTED
    assert lib.joint_attn_fwd_fp8_workspace_bytes(ctypes.byref(bad)) == 0


def test_block_sparse_validation(lib):
    vp = ctypes.c_void_p

    def call(p, mask=FAKE + 0x5000, o=FAKE + 0x3000, q=FAKE):
        return lib.joint_attn_fwd_bf16_block_sparse(
            ctypes.byref(p) if p is not None else None, vp(q), vp(FAKE + 0x1000), KV_BYTES,
            None, vp(mask), vp(o), None, None, 0, None)

    assert call(None) == ja.JA_ERR_INVALID_ARG
    assert call(_p(), mask=0) == ja.JA_ERR_INVALID_ARG                  # mask required
    assert call(_p(), o=FAKE) == ja.JA_ERR_INVALID_ARG                  # o aliases q
    assert call(_p(), q=FAKE + 4) == ja.JA_ERR_INVALID_ARG              # misaligned
    bad = _p()
    bad.head_dim = 96
    assert call(bad) == ja.JA_ERR_UNSUPPORTED
    assert call(_p(s=(1 << 20) + 1)) == ja.JA_ERR_UNSUPPORTED           # longest sequence
    assert ja.block_mask_shape(2, 300, 3) == (2, 3, 3, 5)


def test_prep_kv_validation(lib):
    vp = ctypes.c_void_p
    p = _p(s=300, h=2, d=64)
    need = lib.joint_attn_prep_kv_bf16_bytes(ctypes.byref(p))
    # rotated K and transposed V: 2 tensors x B*H*ceil(S/64)*64*D bf16
    assert need == 2 * 1 * 2 * 320 * 64 * 2
    assert lib.joint_attn_prep_kv_bf16_bytes(None) == 0
    f = lib.joint_attn_prep_kv_bf16
    assert f(None, vp(FAKE), vp(FAKE), None, vp(FAKE + 0x4000), need, None) == ja.JA_ERR_INVALID_ARG
    assert f(ctypes.byref(p), vp(FAKE), vp(FAKE + 0x1000), None, vp(FAKE + 0x4000), need - 16,
             None) == ja.JA_ERR_INVALID_ARG                                # too small
    assert f(ctypes.byref(p), vp(FAKE + 2), vp(FAKE + 0x1000), None, vp(FAKE + 0x4000), need,
             None) == ja.JA_ERR_INVALID_ARG                                # misaligned
    assert f(ctypes.byref(p), vp(FAKE), vp(0), None, vp(FAKE + 0x4000), need,
             None) == ja.JA_ERR_INVALID_ARG
    bad = _p()
    bad.head_dim = 96
    assert f(ctypes.byref(bad), vp(FAKE), vp(FAKE + 0x1000), None, vp(FAKE + 0x4000), need,
             None) == ja.JA_ERR_UNSUPPORTED


def test_norm_validation(lib):
    p = _p()
    p.norm_eps = -1.0
    assert _fwd(lib, p) == ja.JA_ERR_INVALID_ARG
    p = _p()
    p.norm_eps = float("nan")
    assert _fwd(lib, p) == ja.JA_ERR_INVALID_ARG
    p = _p()
    p.q_norm = FAKE + 4                                                 # misaligned weights
    assert _fwd(lib, p) == ja.JA_ERR_INVALID_ARG
    p = _p()
    p.k_norm = FAKE + 8
    vp = ctypes.c_void_p
    assert lib.joint_attn_prep_kv_bf16(ctypes.byref(p), vp(FAKE), vp(FAKE + 0x1000), None,
                                       vp(FAKE + 0x4000), 1 << 30, None) == ja.JA_ERR_INVALID_ARG
