"""The lm_head's argmax helpers and 64-bit keys, built for the host from the
kernels' own header and run on the CPU: the all -inf and NaN cases (row 0,
value -inf), ties to the lowest row, signed zeros, and the key order."""
import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_argmax_keys_on_host(tmp_path):
    exe = str(tmp_path / "argmax_key_check")
    src = os.path.join(ROOT, "tests", "argmax_key_check.cpp")
    cmd = ["/opt/rocm/bin/hipcc", "-x", "hip", "--offload-arch=gfx950", "-O1", "-std=c++17",
           "-I", os.path.join(ROOT, "include"), src, "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    r = subprocess.run([exe], capture_output=True, text=True)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), r.stdout + r.stderr
