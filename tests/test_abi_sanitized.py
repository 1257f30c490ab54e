"""The C ABI tests again, against a host-sanitizer build of the library:
api.cpp (argument validation, launch planning, workspace carving) compiled
with AddressSanitizer and UndefinedBehaviorSanitizer on the host side,
linked with the regular kernel objects, and test_abi.py run in a child
process with the ASan runtime preloaded.  Any sanitizer report fails."""
import importlib.util
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _build_module():
    path = os.path.join(ROOT, "joint_attention_attn_amd", "csrc", "build.py")
    spec = importlib.util.spec_from_file_location("_ja_build_san", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


@pytest.mark.timeout(900)
def test_abi_under_asan_and_ubsan():
    mod = _build_module()
    lib = mod.build_sanitized()
    env = dict(os.environ)
    env["JA_LIBRARY"] = lib
    env["LD_PRELOAD"] = mod.asan_runtime()
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=800)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert " passed" in out
