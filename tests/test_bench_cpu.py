"""bench.py pieces that need no GPU: the single-GPU refusal and the code
digest that ties the committed lm_head counters to the kernel code (bench.py
reports the measured traffic only while the digest matches)."""
import importlib.util
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_code_text_ignores_comments_only():
    b = _bench()
    a = 'int f(int x) { // add one\n  return x + 1; /* done */\n}\n'
    c = 'int f(int x) {\n\n  return x + 1;   \n}\n// trailing note\n'
    assert b.code_text(a) == b.code_text(c)
    assert b.code_text(a) != b.code_text(a.replace("x + 1", "x + 2"))
    # comment markers inside string literals are code
    s = 'const char *p = "a // b";\n'
    assert "// b" in b.code_text(s)

