"""C ABI checks that need no GPU: the library loads, exports every function
that include/joint_attn.h declares, the binding's struct mirrors match the C
layout, and invalid calls are rejected on the host before anything is
enqueued (the pointers below are never dereferenced)."""
import ctypes
import os
import re
import shutil
import subprocess

import pytest

import joint_attention_attn_amd as ja

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "joint_attn.h")
FAKE = 0x10000  # 16-byte aligned stand-in address; validation fails before use
vp = ctypes.c_void_p
INV, UNS = ja.JA_ERR_INVALID_ARG, ja.JA_ERR_UNSUPPORTED


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(ja.library_path()):
        pytest.fail("libjoint_attn.so is not built (run __graft_entry__.build())")
    return ja.load()


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(joint_attn_\w+)\s*\(", text)))


def test_every_declared_symbol_is_exported_and_bound(lib):
    names = _declared()
    assert {"joint_attn_fwd_bf16", "joint_attn_fwd_fp8", "joint_attn_quant_rope_fp8",
            "joint_attn_rope_table_2d", "joint_attn_status_string",
            "joint_attn_fwd_bf16_prepared", "joint_attn_fwd_fp8_prepared",
            "joint_attn_fp8_repair_count"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n
    # the binding declares argument types for every entry point
    assert set(names) == set(ja._SIGNATURES)


def test_struct_layout_matches_the_c_compiler(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no C compiler")
    fields = [f for f, _ in ja.Params._fields_]
    src = ['#include <stdio.h>', '#include <stddef.h>', f'#include "{HEADER}"', "int main(void) {",
           'printf("%zu\\n", sizeof(ja_params));']
    src += [f'printf("%zu\\n", offsetof(ja_params, {f}));' for f in fields]
    src += ['printf("%zu\\n", sizeof(ja_fp8_repair));']
    src += [f'printf("%zu\\n", offsetof(ja_fp8_repair, {f}));' for f, _ in ja.Fp8RepairC._fields_]
    src += ["return 0; }"]
    (tmp_path / "layout.c").write_text("\n".join(src))
    exe = tmp_path / "layout"
    subprocess.run([gcc, "-std=c99", "-Wall", "-Werror", str(tmp_path / "layout.c"), "-o", str(exe)],
                   check=True)
    got = [int(x) for x in subprocess.run([str(exe)], capture_output=True, text=True,
                                          check=True).stdout.split()]
    want = [ctypes.sizeof(ja.Params)] + [getattr(ja.Params, f).offset for f in fields]
    want += [ctypes.sizeof(ja.Fp8RepairC)] + [getattr(ja.Fp8RepairC, f).offset
                                             for f, _ in ja.Fp8RepairC._fields_]
    assert got == want


def test_status_strings_and_last_error(lib):
    for code in range(4):
        assert lib.joint_attn_status_string(code).startswith(b"JA_")
    assert lib.joint_attn_status_string(99) == b"unknown ja_status"
    bad = _p()
    bad.head_dim = 96
    assert _fwd(lib, bad) == UNS
    assert b"head_dim 96" in lib.joint_attn_last_error()


def _p(b=1, s=80, h=2, d=64):
    p = ja.Params(b, s, h, d)
    for x in "qkvo":
        setattr(p, f"{x}_sb", s * h * d)
        setattr(p, f"{x}_ss", h * d)
        setattr(p, f"{x}_sh", d)
    return p


BIG = 1 << 30   # stand-in size of buffers and workspaces


def _fwd(lib, p, q=FAKE, k=FAKE + 0x1000, v=FAKE + 0x2000, o=FAKE + 0x3000, lse=None,
         ws=FAKE + 0x8000, ws_bytes=BIG):
    return lib.joint_attn_fwd_bf16(ctypes.byref(p) if p is not None else None, vp(q), vp(k),
                                   vp(v), vp(o), vp(lse), vp(ws), ws_bytes, None)


@pytest.mark.parametrize("mutate,expect", [
    (lambda p: setattr(p, "batch", 0), INV),
    (lambda p: setattr(p, "seq_len", 0), INV),
    (lambda p: setattr(p, "heads", -1), INV),
    (lambda p: setattr(p, "head_dim", 96), UNS),
    (lambda p: setattr(p, "head_dim", 256), UNS),
    (lambda p: setattr(p, "q_ss", 100), INV),
    (lambda p: setattr(p, "k_sh", 4), INV),
    (lambda p: setattr(p, "v_sb", 12), INV),
    (lambda p: setattr(p, "o_sb", -8), INV),
    (lambda p: setattr(p, "softmax_scale", float("nan")), INV),
    (lambda p: setattr(p, "softmax_scale", -1.0), INV),
    (lambda p: setattr(p, "heads", 70000), UNS),
    (lambda p: setattr(p, "rope_theta", -1.0), INV),
    (lambda p: setattr(p, "rope_theta", float("inf")), INV),
    (lambda p: setattr(p, "pos", FAKE + 2), INV),                 # misaligned positions
    (lambda p: setattr(p, "rope_table", FAKE + 8), INV),          # misaligned table
    (lambda p: setattr(p, "flags", 6), INV),
])
def test_fwd_bf16_rejects_bad_params(lib, mutate, expect):
    p = _p()
    mutate(p)
    if p.rope_table:
        p.rope_table_bytes = BIG
    assert _fwd(lib, p) == expect


def test_rope_table_size_is_checked(lib):
    # a table built for fewer tokens or head_dim 64 instead of 128 is refused
    p = _p(s=80, d=128)
    p.rope_table = FAKE + 0x10000
    p.rope_table_bytes = 80 * 128 * 8 - 1
    assert _fwd(lib, p) == INV
    assert b"rope_table_bytes" in lib.joint_attn_last_error()
    p.rope_table_bytes = 80 * 64 * 8
    assert _fwd(lib, p) == INV
    p.rope_table_bytes = 80 * 128 * 8
    assert lib.joint_attn_fwd_bf16_workspace_bytes(ctypes.byref(p)) > 0


def test_fwd_bf16_rejects_bad_pointers(lib):
    assert _fwd(lib, None) == INV
    assert _fwd(lib, _p(), q=0) == INV
    assert _fwd(lib, _p(), k=0) == INV
    assert _fwd(lib, _p(), o=0) == INV
    assert _fwd(lib, _p(), v=FAKE + 0x2002) == INV                   # misaligned
    assert _fwd(lib, _p(), lse=FAKE + 2) == INV
    assert _fwd(lib, _p(), o=FAKE) == INV                            # o aliases q
    assert _fwd(lib, _p(), ws=FAKE + 0x8008) == INV                  # misaligned workspace
    assert _fwd(lib, _p(), ws=0) == INV                              # workspace required
    need = lib.joint_attn_fwd_bf16_workspace_bytes(ctypes.byref(_p()))
    assert _fwd(lib, _p(), ws_bytes=need - 1) == INV
    assert b"workspace" in lib.joint_attn_last_error()


def test_workspace_sizes(lib):
    p = _p(s=300, h=2, d=64)
    kv = 2 * 1 * 2 * 320 * 64 * 2             # rotated K and V^T, S_pad = 320
    # no RoPE, or a table given: K/V only; positions alone: K/V plus the
    # table and the coordinate table (1024 coordinates x D/4 pairs x 16 B)
    assert lib.joint_attn_prep_kv_bf16_bytes(ctypes.byref(p)) == kv
    p.pos = FAKE
    assert lib.joint_attn_prep_kv_bf16_bytes(ctypes.byref(p)) == \
        kv + (300 * 64 * 8 + 255) // 256 * 256 + 1024 * 16 * 16
    assert lib.joint_attn_quant_rope_fp8_workspace_bytes(ctypes.byref(p)) == 300 * 64 * 8
    assert lib.joint_attn_fp8_repair_plan_workspace_bytes(ctypes.byref(p)) == 300 * 64 * 8
    p.rope_table, p.rope_table_bytes = FAKE + 0x1000, 300 * 64 * 8
    assert lib.joint_attn_prep_kv_bf16_bytes(ctypes.byref(p)) == kv
    assert lib.joint_attn_quant_rope_fp8_workspace_bytes(ctypes.byref(p)) == 0
    # the one-call forward: prepared K/V plus the split's partial results
    for f in (lib.joint_attn_fwd_bf16_workspace_bytes,):
        assert f(ctypes.byref(p)) == kv + lib.joint_attn_fwd_bf16_prepared_workspace_bytes(
            ctypes.byref(p))
    n8 = lib.joint_attn_prep_kv_fp8_bytes(ctypes.byref(p))
    assert lib.joint_attn_fwd_fp8_workspace_bytes(ctypes.byref(p)) == (n8 + 255) // 256 * 256 + \
        lib.joint_attn_fwd_fp8_prepared_workspace_bytes(ctypes.byref(p))
    # invalid parameters: 0
    for f in (lib.joint_attn_fwd_bf16_workspace_bytes, lib.joint_attn_prep_kv_bf16_bytes,
              lib.joint_attn_fwd_bf16_prepared_workspace_bytes,
              lib.joint_attn_quant_rope_fp8_workspace_bytes,
              lib.joint_attn_fwd_fp8_workspace_bytes, lib.joint_attn_prep_kv_fp8_bytes,
              lib.joint_attn_fwd_fp8_prepared_workspace_bytes,
              lib.joint_attn_fp8_repair_plan_workspace_bytes):
        assert f(None) == 0
        bad = _p()
        bad.head_dim = 96
        assert f(ctypes.byref(bad)) == 0


def test_rope_table_validation(lib):
    f = lib.joint_attn_rope_table_2d
    assert f(vp(0), 10, 64, 10000.0, vp(FAKE), None) == INV
    assert f(vp(FAKE), 0, 64, 10000.0, vp(FAKE), None) == INV
    assert f(vp(FAKE), 10, 64, 0.0, vp(FAKE), None) == INV
    assert f(vp(FAKE), 10, 64, float("inf"), vp(FAKE), None) == INV
    assert f(vp(FAKE), 10, 48, 10000.0, vp(FAKE), None) == UNS
    assert f(vp(FAKE), 10, 64, 10000.0, vp(FAKE + 4), None) == INV


def _prepared(lib, p, q=FAKE, kv=FAKE + 0x1000, kv_bytes=BIG, o=FAKE + 0x3000, lse=None,
              ws=None, ws_bytes=0):
    return lib.joint_attn_fwd_bf16_prepared(ctypes.byref(p) if p is not None else None, vp(q),
                                            vp(kv), kv_bytes, vp(o), vp(lse), vp(ws), ws_bytes,
                                            None)


def test_prepared_forward_validation(lib):
    assert _prepared(lib, None) == INV
    assert _prepared(lib, _p(), q=0) == INV
    assert _prepared(lib, _p(), kv=0) == INV
    assert _prepared(lib, _p(), kv=FAKE + 0x1002) == INV
    assert _prepared(lib, _p(), kv_bytes=1024) == INV                  # too small
    assert _prepared(lib, _p(), o=FAKE) == INV                         # aliases q
    assert _prepared(lib, _p(), o=FAKE + 0x1000) == INV                # aliases kv
    assert _prepared(lib, _p(), ws=FAKE + 0x4008, ws_bytes=64) == INV  # misaligned
    p = _p()
    p.pos = FAKE
    need = lib.joint_attn_prep_kv_bf16_bytes(ctypes.byref(p))
    assert _prepared(lib, p, kv_bytes=need - 16) == INV               # the table is part of kv


def test_prep_kv_validation(lib):
    p = _p(s=300, h=2, d=64)
    need = lib.joint_attn_prep_kv_bf16_bytes(ctypes.byref(p))
    f = lib.joint_attn_prep_kv_bf16
    assert f(None, vp(FAKE), vp(FAKE), vp(FAKE + 0x4000), need, None) == INV
    assert f(ctypes.byref(p), vp(FAKE), vp(FAKE + 0x1000), vp(FAKE + 0x4000), need - 16,
             None) == INV                                                 # too small
    assert f(ctypes.byref(p), vp(FAKE + 2), vp(FAKE + 0x1000), vp(FAKE + 0x4000), need,
             None) == INV                                                 # misaligned
    assert f(ctypes.byref(p), vp(FAKE), vp(0), vp(FAKE + 0x4000), need, None) == INV
    bad = _p()
    bad.head_dim = 96
    assert f(ctypes.byref(bad), vp(FAKE), vp(FAKE + 0x1000), vp(FAKE + 0x4000), need,
             None) == UNS


def _quant(lib, p, ptrs=None, ws=None, ws_bytes=0):
    ptrs = ptrs or [vp(FAKE + 0x1000 * i) for i in range(9)]
    return lib.joint_attn_quant_rope_fp8(ctypes.byref(p), *ptrs, vp(ws), ws_bytes, None)


def test_quant_validation(lib):
    bad = _p()
    bad.head_dim = 32
    assert _quant(lib, bad) == UNS
    ptrs = [vp(FAKE + 0x1000 * i) for i in range(9)]
    assert _quant(lib, _p(), [vp(0)] + ptrs[1:]) == INV
    assert _quant(lib, _p(), ptrs[:6] + [vp(FAKE + 0x6002)] + ptrs[7:]) == INV   # misaligned sq
    p = _p()
    p.q_sh = 4
    assert _quant(lib, p) == INV
    # positions without a table: the workspace holds the table
    p = _p()
    p.pos = FAKE
    assert _quant(lib, p) == INV
    assert _quant(lib, p, ws=FAKE + 0x20000, ws_bytes=80 * 64 * 8 - 8) == INV


def _fwd8(lib, p, q8=FAKE, k8=FAKE + 0x1000, v8=FAKE + 0x2000, sq=FAKE + 0x3000,
          sk=FAKE + 0x4000, sv=FAKE + 0x5000, o=FAKE + 0x6000, lse=None, ws=FAKE + 0x8000,
          ws_bytes=BIG):
    return lib.joint_attn_fwd_fp8(ctypes.byref(p), vp(q8), vp(k8), vp(v8), vp(sq), vp(sk), vp(sv),
                                  vp(o), vp(lse), vp(ws), ws_bytes, None)


def _fwd8p(lib, p, q8=FAKE, sq=FAKE + 0x1000, kv8=FAKE + 0x2000, kv8_bytes=BIG, rep=None,
           o=FAKE + 0x3000, lse=None, ws=None, ws_bytes=0):
    return lib.joint_attn_fwd_fp8_prepared(ctypes.byref(p), vp(q8), vp(sq), vp(kv8), kv8_bytes,
                                           ctypes.byref(rep) if rep is not None else None, vp(o),
                                           vp(lse), vp(ws), ws_bytes, None)


def _prep8(lib, p, k8=FAKE, v8=FAKE + 0x1000, sk=FAKE + 0x2000, sv=FAKE + 0x3000, rep=None,
           kv8=FAKE + 0x4000, kv8_bytes=BIG):
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
    assert _prep8(lib, bad) == UNS
    assert _prep8(lib, p, k8=0) == INV
    assert _prep8(lib, p, sk=FAKE + 0x2002) == INV
    assert _prep8(lib, p, kv8=FAKE + 0x4004) == INV
    assert _prep8(lib, p, kv8_bytes=n - 1) == INV
    assert _prep8(lib, p, rep=ja.Fp8RepairC(5, None, FAKE, FAKE)) == INV
    assert _prep8(lib, p, rep=ja.Fp8RepairC(81, FAKE, FAKE, FAKE)) == INV
    assert _prep8(lib, p, rep=ja.Fp8RepairC(-1, FAKE, FAKE, FAKE)) == INV

    assert _fwd8p(lib, bad) == UNS
    assert _fwd8p(lib, p, q8=FAKE + 4) == INV
    assert _fwd8p(lib, p, sq=FAKE + 0x1002) == INV
    assert _fwd8p(lib, p, o=0) == INV
    assert _fwd8p(lib, p, o=FAKE) == INV                               # aliases q8
    assert _fwd8p(lib, p, kv8_bytes=n - 1) == INV
    assert _fwd8p(lib, p, ws=FAKE + 0x9008, ws_bytes=64) == INV
    assert _fwd8p(lib, p, rep=ja.Fp8RepairC(5, FAKE, None, FAKE)) == INV
    assert _fwd8p(lib, p, rep=ja.Fp8RepairC(81, FAKE, FAKE, FAKE)) == INV

    assert _fwd8(lib, bad) == UNS
    assert _fwd8(lib, p, k8=0) == INV
    assert _fwd8(lib, p, sk=FAKE + 0x4002) == INV
    assert _fwd8(lib, p, o=FAKE + 0x2000) == INV                        # aliases v8
    assert _fwd8(lib, p, ws=0) == INV
    need = lib.joint_attn_fwd_fp8_workspace_bytes(ctypes.byref(p))
    assert _fwd8(lib, p, ws_bytes=need - 1) == INV


def test_repair_count(lib):
    f = lib.joint_attn_fp8_repair_count
    assert f(0.005, 16896) == 85 and f(0.005, 80) == 1
    assert f(0.0, 80) == 0 and f(1.0, 80) == 80
    assert f(-0.1, 80) == -1 and f(1.5, 80) == -1 and f(float("nan"), 80) == -1
    assert f(0.5, 0) == -1
    assert ja.repair_count(0.005, 16896) == 85
    with pytest.raises(ja.JointAttnError):
        ja.repair_count(2.0, 10)


def test_repair_plan_validation(lib):
    p = _p()
    ptrs = [vp(FAKE + 0x1000 * i) for i in range(12)]
    f = lib.joint_attn_fp8_repair_plan

    def call(pp, n, idx=ptrs[6], ws=None, ws_bytes=0):
        return f(ctypes.byref(pp), *ptrs[:6], n, idx, *ptrs[7:10], vp(ws), ws_bytes, None)

    assert call(p, 81) == INV
    assert call(p, -1) == INV
    assert call(p, 4, idx=None) == INV
    assert call(_p(s=40000), 4) == UNS
    bad = _p()
    bad.head_dim = 96
    assert call(bad, 4) == UNS
    pp = _p()
    pp.pos = FAKE
    assert call(pp, 4) == INV                                           # the table needs a workspace


def test_block_sparse_validation(lib):
    def call(p, mask=FAKE + 0x5000, o=FAKE + 0x3000, q=FAKE):
        return lib.joint_attn_fwd_bf16_block_sparse(
            ctypes.byref(p) if p is not None else None, vp(q), vp(FAKE + 0x1000),
            vp(FAKE + 0x2000), vp(mask), vp(o), None, vp(FAKE + 0x8000), BIG, None)

    def call_prepared(p, mask=FAKE + 0x5000):
        return lib.joint_attn_fwd_bf16_block_sparse_prepared(
            ctypes.byref(p), vp(FAKE), vp(FAKE + 0x1000), BIG, vp(mask), vp(FAKE + 0x3000), None,
            None, 0, None)

    assert call(None) == INV
    assert call(_p(), mask=0) == INV                                    # mask required
    assert call_prepared(_p(), mask=0) == INV
    assert call(_p(), o=FAKE) == INV                                    # o aliases q
    assert call(_p(), q=FAKE + 4) == INV                                # misaligned
    bad = _p()
    bad.head_dim = 96
    assert call(bad) == UNS
    assert call(_p(s=(1 << 20) + 1)) == UNS                             # longest sequence
    assert call_prepared(_p(s=(1 << 20) + 1)) == UNS
    assert ja.block_mask_shape(2, 300, 3) == (2, 3, 3, 5)


def test_fp8_block_sparse_validation(lib):
    def call(p, mask=FAKE + 0x7000, o=FAKE + 0x6000):
        return lib.joint_attn_fwd_fp8_block_sparse(
            ctypes.byref(p), vp(FAKE), vp(FAKE + 0x1000), vp(FAKE + 0x2000), vp(FAKE + 0x3000),
            vp(FAKE + 0x4000), vp(FAKE + 0x5000), vp(mask), vp(o), None, vp(FAKE + 0x8000), BIG,
            None)

    def call_prepared(p, mask=FAKE + 0x7000):
        return lib.joint_attn_fwd_fp8_block_sparse_prepared(
            ctypes.byref(p), vp(FAKE), vp(FAKE + 0x1000), vp(FAKE + 0x2000), BIG, vp(mask),
            vp(FAKE + 0x6000), None, None, 0, None)

    assert call(_p(), mask=0) == INV
    assert call_prepared(_p(), mask=0) == INV
    assert call(_p(), o=FAKE) == INV                                    # o aliases q8
    assert call(_p(s=(1 << 20) + 1)) == UNS
    assert call_prepared(_p(s=(1 << 20) + 1)) == UNS
    bad = _p()
    bad.head_dim = 96
    assert call(bad) == UNS


def test_norm_validation(lib):
    p = _p()
    p.norm_eps = -1.0
    assert _fwd(lib, p) == INV
    p = _p()
    p.norm_eps = float("nan")
    assert _fwd(lib, p) == INV
    p = _p()
    p.q_norm = FAKE + 4                                                 # misaligned weights
    assert _fwd(lib, p) == INV
    p = _p()
    p.k_norm = FAKE + 8
    assert lib.joint_attn_prep_kv_bf16(ctypes.byref(p), vp(FAKE), vp(FAKE + 0x1000),
                                       vp(FAKE + 0x4000), BIG, None) == INV


def test_binding_rejects_wrong_tensors():
    # dtype, shape and device checks in the binding run before any library
    # call (CPU tensors are not device tensors)
    import torch
    q = torch.zeros((1, 8, 2, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        ja.fwd_bf16(q, q, q)                          # not on a device
    with pytest.raises(ValueError):
        ja.rope_table_2d(torch.zeros((8, 2), dtype=torch.int32), 64)
