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



def test_kernel_class_names():
    b = _bench()
    kc = b.kernel_class
    assert kc("mv::lmhead_kernel<false>(...)") == "lm_bf16"
    assert kc("void mv::lmhead_kernel<true>(int)") == "lm_fp8"
    assert kc("mv::expert_up_kernel<5, false, true, true>") == "up_bf16"
    assert kc("mv::expert_up_kernel<3, true, false, true>") == "up_fp8"
    assert kc("mv::expert_down_gemv_kernel<10, false, 8>") == "down_bf16"
    assert kc("mv::expert_down_gemv_kernel<10, true, 12>") == "down_fp8"
    assert kc("mv::expert_down_kernel<10, 1, 8>") == "down_bf16"
    assert kc("mv::route_kernel<2, 0, 8, 2, false, 8, 4>") == "route_partials"
    assert kc("mv::route_kernel<2, 8, 8, 2, false, 8, 4>") == "route"
    assert kc("mv::route_kernel<2, 8, 8, 2, true, 8, 4>") == "route_norm"
    assert kc("at::native::bitwise_not_kernel") == "calib"
    assert kc("mv::fill_zero_kernel(...)") is None


def test_counter_summary_from_csv(tmp_path):
    """Two fabricated counter files: the calibration kernel sets the scale
    (FETCH_SIZE reads half the bytes, WRITE_SIZE all), the lm_head's bytes
    follow from it and are set against the algorithmic bytes given."""
    import csv
    import json
    b = _bench()
    cal = 1024 * 2**20
    rows = {"FETCH_SIZE": [("void at::native::bitwise_not_kernel(int)", cal / 2 / 1024),
                           ("void mv::lmhead_kernel<false>(int)", 1000.0),
                           ("void mv::lmhead_kernel<false>(int)", 1002.0)],
            "WRITE_SIZE": [("void at::native::bitwise_not_kernel(int)", cal / 1024),
                           ("void mv::lmhead_kernel<false>(int)", 4.0),
                           ("void mv::lmhead_kernel<false>(int)", 4.0)]}
    paths = []
    for counter, rs in rows.items():
        p = tmp_path / f"{counter}.csv"
        with open(p, "w", newline="") as f:
            w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
            w.writeheader()
            for name, v in rs:
                w.writerow({"Kernel_Name": name, "Counter_Name": counter, "Counter_Value": v})
        paths.append(str(p))
    algo = tmp_path / "algo.json"
    algo.write_text(json.dumps({"workload": "t", "M": 1, "definition": "d",
                                "classes": {"lm_bf16": {"read": 2002 * 1024, "write": 8}}}))

    class A:
        write_counters = paths
        calib_mib = 1024
        title = "t"
        cmd = ["c"]

    A.algo = str(algo)
    A.out = "zz_test_summary.md"
    out = os.path.join(b.PROFILES, A.out)
    try:
        b.write_counters(A)
        text = open(out).read()
    finally:
        if os.path.exists(out):
            os.remove(out)
    # 1001 KiB mean at factor 0.5 -> 2002 KiB of HBM reads, ratio 1.0000
    assert "| lmhead_kernel<false> | 2 | 1001.0 | 2,050,048 | 2,050,048 | 1.0000 |" in text
