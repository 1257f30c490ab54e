"""Host-side behaviour of bench.py that needs no GPU."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    # the benchmark measures one GPU; --gpus 2 (or a WORLD_SIZE above 1)
    # exits with status 2 and says so, before touching any device
    for args, env in ((["--gpus", "2"], {}), (["--gpus", "1"], {"WORLD_SIZE": "2"})):
        r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                           capture_output=True, text=True, timeout=60,
                           env={**os.environ, **env})
        assert r.returncode == 2
        assert "more than one GPU" in r.stderr
        assert r.stdout == ""
