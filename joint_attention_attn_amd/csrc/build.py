"""Build libjoint_attn.so for gfx950 with hipcc (in-tree).

Each source compiles to an object in parallel, then hipcc links the shared
library next to the Python binding.  Always rebuilds: the build is the
"does it compile" check as well as the product build.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
PKG = os.path.dirname(HERE)
LIB = os.path.join(PKG, "libjoint_attn.so")
SOURCES = ["api.cpp", "rope_table.hip", "prep_kv.hip", "attn_bf16.hip", "split.hip", "quant_fp8.hip", "prep_kv_fp8.hip", "attn_fp8.hip", "repair_fp8.hip"]
ARCH = "gfx950"
# Packed-fp32 VALU forms are left to nobody: the compiler may not emit them.
FLAGS = ["-O3", "-std=c++20", "-fPIC", f"--offload-arch={ARCH}",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-command-line-argument"]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else (shutil.which("hipcc") or "hipcc")


def build(verbose: bool = False, extra_flags=None) -> str:
    out_dir = os.path.join(PKG, "_build")
    os.makedirs(out_dir, exist_ok=True)
    flags = FLAGS + list(extra_flags or [])
    cc = hipcc()

    def compile_one(src):
        obj = os.path.join(out_dir, os.path.splitext(src)[0] + ".o")
        cmd = [cc, *flags, "-c", os.path.join(HERE, src), "-o", obj]
        if src.endswith(".cpp"):
            cmd[1:1] = ["-x", "hip"]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
        if verbose and r.stderr.strip():
            print(r.stderr)
        return obj

    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIB + ".tmp"
    r = subprocess.run([cc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    build_probe(cc, out_dir)
    return LIB


# Stand-alone microbenchmark of the bf16 forward's per-tile instruction chain
# (mfma_chain_probe.hip): the rate the chip sustains for that mix of matrix,
# vector and LDS work under its power limit.  Not part of the library.
PROBE = os.path.join(PKG, "_build", "mfma_chain_probe")


def build_probe(cc: str, out_dir: str) -> str:
    r = subprocess.run([cc, *FLAGS, os.path.join(HERE, "mfma_chain_probe.hip"), "-o", PROBE],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on mfma_chain_probe.hip:\n{r.stdout}\n{r.stderr}")
    return PROBE


# Host-side AddressSanitizer + UndefinedBehaviorSanitizer build of the C ABI
# layer (api.cpp: argument validation, planning, workspace carving), linked
# with the kernel objects of the regular build.  Device code is not
# instrumented (-Xarch_host).  Loading it needs the ASan runtime preloaded.
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=undefined",
             "-Xarch_host", "-fno-omit-frame-pointer", "-g"]


def asan_runtime() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    base = os.path.join(rocm, "lib", "llvm", "lib", "clang")
    for ver in sorted(os.listdir(base), reverse=True):
        path = os.path.join(base, ver, "lib", "linux", "libclang_rt.asan-x86_64.so")
        if os.path.exists(path):
            return path
    raise RuntimeError("no libclang_rt.asan-x86_64.so under " + base)


def build_sanitized() -> str:
    out_dir = os.path.join(PKG, "_build")
    objs = [os.path.join(out_dir, os.path.splitext(src)[0] + ".o") for src in SOURCES
            if src != "api.cpp"]
    if not all(os.path.exists(o) for o in objs):
        build()
    cc = hipcc()
    api_o = os.path.join(out_dir, "api_san.o")
    r = subprocess.run([cc, "-x", "hip", *FLAGS, *SAN_FLAGS, "-c", os.path.join(HERE, "api.cpp"),
                        "-o", api_o], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"sanitized api.cpp failed:\n{r.stdout}\n{r.stderr}")
    lib = os.path.join(out_dir, "libjoint_attn_san.so")
    r = subprocess.run([cc, "-shared", "-fPIC", f"--offload-arch={ARCH}", api_o, *objs,
                        "-o", lib], capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"sanitized link failed:\n{r.stdout}\n{r.stderr}")
    return lib


if __name__ == "__main__":
    print(build(verbose=True))
