#!/usr/bin/env python3
"""Cold-weight bench of the batch-1 MoE verify hot path on one MI355X.

One step = one pass of the whole path over one batch of M verify tokens:
  moe_layer     router gate GEMV + softmax top-k, then the selected experts'
                SwiGLU FFN with weighted combine (one MoE layer verify step)
  lmhead_greedy_verify
                lm_head GEMV fused with the greedy argmax and the greedy
                verdict of the verify chain (accept length, bonus token)
Weights are seeded synthetic bf16 ~N(0, 0.02) generated on the device: 16
distinct MoE layers (8.06 GB each) rotated step by step and two lm_head
copies (805 MB each) alternated, so every weight byte comes from HBM (the
gap between two visits of the same bytes is far beyond the 256 MB of
Infinity Cache plus L2).

Prints ONE JSON line. `value` is the MoE layer's algorithmic bytes per
layer-step / its time (GB/s) at M = 6, where algorithmic bytes = the router
gate, every distinct selected expert's weights once, and the activations and
outputs; the lm_head, the other widths, the graph replay, the coldness
sweeps and the CPU oracle are their own records in the same line.
"""
from __future__ import annotations

import argparse
import csv
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, published
PROFILES = os.path.join(ROOT, "profiles")


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=64)
    ap.add_argument("--warmup", type=int, default=16)
    ap.add_argument("--M", type=int, default=6)
    ap.add_argument("--layers", type=int, default=16, help="distinct MoE layers rotated")
    ap.add_argument("--lm-copies", type=int, default=2)
    ap.add_argument("--fp8-layers", type=int, default=8,
                    help="distinct fp8 expert layers rotated for the fp8 lines (0 skips them)")
    ap.add_argument("--router-copies", type=int, default=512,
                    help="distinct router gates rotated in the gate-only timing")
    ap.add_argument("--zipf-alpha", type=float, default=None,
                    help="add a Zipf(1.1)-shaped router bias of this strength")
    ap.add_argument("--graph-steps", type=int, default=16,
                    help="steps captured in one HIP graph for the replay timing (0 skips it)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-reps", type=int, default=3, help="CPU oracle: best of this many")
    ap.add_argument("--profile-steps", type=int, default=0,
                    help="only run this many steps (for rocprofv3), print nothing else")
    ap.add_argument("--identical-tokens", action="store_true",
                    help="profile mode: every verify token is the same row (the M = 1 routing)")
    ap.add_argument("--algo-out", default=None,
                    help="profile mode: write the algorithmic bytes of every kernel class "
                         "(mean per call) to this JSON file")
    ap.add_argument("--calib-mib", type=int, default=1024,
                    help="profile mode: size of the int32 bitwise_not calibration kernel "
                         "(reads and writes this many MiB)")
    ap.add_argument("--write-counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="no GPU: turn two rocprofv3 --pmc counter_collection.csv files "
                         "(FETCH_SIZE run, WRITE_SIZE run) of the profile mode into HBM bytes "
                         "per kernel (needs --algo and --out)")
    ap.add_argument("--write-stats", metavar="KERNEL_STATS_CSV",
                    help="no GPU: turn one rocprofv3 --stats kernel_stats.csv of the profile "
                         "mode into a table of average kernel durations (needs --algo, --out)")
    ap.add_argument("--algo", default=None, help="the --algo-out file of the profiled run")
    ap.add_argument("--out", default=None, help="summary file to write under profiles/")
    ap.add_argument("--title", default="", help="summary title")
    ap.add_argument("--cmd", action="append", default=[],
                    help="a command that made the profiled data (repeatable)")
    return ap.parse_args()


# ------------------------------------------------------------ source digest

def code_text(src: str) -> str:
    """C++ source without comments and blank-line or trailing-space
    differences: what the compiler sees of it."""
    out, i, n = [], 0, len(src)
    while i < n:
        if src.startswith("//", i):
            i = src.find("\n", i)
            i = n if i < 0 else i
        elif src.startswith("/*", i):
            j = src.find("*/", i + 2)
            i = n if j < 0 else j + 2
        elif src[i] == '"':                     # string literals are kept whole
            j = i + 1
            while j < n and src[j] != '"':
                j += 2 if src[j] == "\\" else 1
            out.append(src[i:j + 1])
            i = j + 1
        else:
            out.append(src[i])
            i += 1
    lines = [ln.rstrip() for ln in "".join(out).splitlines()]
    return "\n".join(ln for ln in lines if ln)


def src_digest(*names: str) -> str:
    """Digest of the code (not the comments) of the named sources: the
    counters stay valid while it matches."""
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "moe_speculative_verify_amd", "csrc", n)) as f:
            h.update(code_text(f.read()).encode())
    return h.hexdigest()[:16]


LM_DIGEST_SOURCES = ("lmhead.hip", "common.h")
ALL_SOURCES = ("common.h", "select.h", "route.hip", "expert.hip", "lmhead.hip", "capi.hip")


# ------------------------------------------------- profile summaries (no GPU)

CALIB_KERNEL = "bitwise_not"     # substring of the calibration kernel's name


def kernel_class(name: str) -> str | None:
    """The class of a kernel name in a rocprofv3 file: which algorithmic
    byte count applies to it."""
    import re
    m = re.search(r"(\w+)<([^>]*)>", name)
    if not m:
        return "calib" if CALIB_KERNEL in name else None
    base, targs = m.group(1), [a.strip() for a in m.group(2).split(",")]
    if base == "lmhead_kernel":
        return "lm_fp8" if targs[0] == "true" else "lm_bf16"
    if base == "expert_up_kernel":
        return "up_fp8" if targs[1] == "true" else "up_bf16"
    if base == "expert_down_gemv_kernel":
        return "down_fp8" if targs[1] == "true" else "down_bf16"
    if base == "expert_down_kernel":
        return "down_bf16"
    if base == "route_kernel":
        # route_kernel<S, KJ, RT, P, NORM, W, KS>: KJ = 0 writes partial
        # logits only (the layer's router; selection happens in the up kernel)
        if targs[4] == "true":
            return "route_norm"
        return "route_partials" if targs[1] == "0" else "route"
    if base == "fill_zero_kernel" or base == "hbm_read_kernel":
        return None
    return None


def short_name(name: str) -> str:
    i = name.find("(")
    name = name if i < 0 else name[:i]
    return name.replace("void ", "").replace("mv::", "").strip()


def read_counter_rows(path: str, counter: str) -> dict:
    """Per kernel name: the per-dispatch values of `counter` in one
    rocprofv3 counter_collection.csv."""
    vals: dict = {}
    with open(path, newline="") as f:
        for row in csv.DictReader(f):
            if row.get("Counter_Name") != counter:
                continue
            vals.setdefault(short_name(row.get("Kernel_Name", "")), []).append(
                float(row["Counter_Value"]))
    return vals


def write_counters(args) -> None:
    """FETCH_SIZE and WRITE_SIZE (KiB per dispatch) of every kernel of a
    profile run, each scaled by what the same counter reads for the
    calibration kernel (calib_mib MiB in and out): bytes = KiB * 1024 / factor,
    set against the algorithmic bytes the profile run logged."""
    if not (args.algo and args.out):
        raise SystemExit("--write-counters needs --algo and --out")
    fe = read_counter_rows(args.write_counters[0], "FETCH_SIZE")
    wr = read_counter_rows(args.write_counters[1], "WRITE_SIZE")
    with open(args.algo) as f:
        algo = json.load(f)
    cal = [k for k in fe if CALIB_KERNEL in k]
    calw = [k for k in wr if CALIB_KERNEL in k]
    if not cal or not calw:
        raise SystemExit("no calibration kernel rows in the counter files")
    calib_bytes = args.calib_mib * 2**20
    f_fac = sum(fe[cal[0]]) / len(fe[cal[0]]) * 1024 / calib_bytes
    w_fac = sum(wr[calw[0]]) / len(wr[calw[0]]) * 1024 / calib_bytes
    rows = []
    for name in sorted(fe):
        cls = kernel_class(name)
        if cls is None or cls == "calib" or name not in wr:
            continue
        f_kib = sum(fe[name]) / len(fe[name])
        w_kib = sum(wr[name]) / len(wr[name])
        a = algo["classes"].get(cls, {})
        rows.append(dict(kernel=name, cls=cls, dispatches=len(fe[name]), fetch_kib=f_kib,
                         read_b=f_kib * 1024 / f_fac, algo_read_b=a.get("read"),
                         write_kib=w_kib, write_b=w_kib * 1024 / w_fac,
                         algo_write_b=a.get("write")))
    lines = [f"# {args.title}" if args.title else "# rocprofv3 HBM counters",
             "# commands (repository root on the machine with the GPU, TMPDIR=/tmp), one counter pass each:"]
    lines += [f"#   {c}" for c in args.cmd]
    lines += [f"# summary: python3 bench.py --write-counters <fetch csv> <write csv> "
              f"--algo <algo json> --out {os.path.basename(args.out)}",
              f"# source digest (code of {', '.join(ALL_SOURCES)}): {src_digest(*ALL_SOURCES)}",
              "", f"Workload: {algo['workload']}.",
              "Distinct experts per expert call (mean): " + (", ".join(
                  f"{kd} {sum(v) / len(v):.2f} over {len(v)} calls"
                  for kd, v in algo.get("distinct_experts", {}).items()) or "none") + ".",
              f"Counter to bytes: FETCH_SIZE x 1024 / {f_fac:.4f}, WRITE_SIZE x 1024 / "
              f"{w_fac:.4f} (the factors the calibration kernel, torch int32 bitwise_not over "
              f"{args.calib_mib} MiB in and out, reads in the same runs).",
              "Algorithmic bytes per call (mean): " + algo["definition"], "",
              "| kernel | dispatches | FETCH_SIZE KiB | HBM read B | algorithmic read B | ratio "
              "| WRITE_SIZE KiB | HBM write B | algorithmic write B |",
              "|---|---|---|---|---|---|---|---|---|"]
    for r in rows:
        ar, aw = r["algo_read_b"], r["algo_write_b"]
        ratio = f"{r['read_b'] / ar:.4f}" if ar else "—"
        lines.append(f"| {r['kernel']} | {r['dispatches']} | {r['fetch_kib']:.1f} | "
                     f"{r['read_b']:,.0f} | {f'{ar:,.0f}' if ar else '—'} | {ratio} | "
                     f"{r['write_kib']:.1f} | {r['write_b']:,.0f} | "
                     f"{f'{aw:,.0f}' if aw else '—'} |")
    path = os.path.join(PROFILES, os.path.basename(args.out))
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    # the lm_head's counters feed the bench line's roofline.traffic
    lm = [r for r in rows if r["cls"] == "lm_bf16"]
    if lm and algo.get("M") == 6 and not algo.get("identical_tokens"):
        r = lm[0]
        with open(os.path.join(PROFILES, "lmhead_argmax_counters.json"), "w") as f:
            json.dump({"kernel": r["kernel"] + ", 157184x2560 bf16, M=6",
                       "source_digest": src_digest(*LM_DIGEST_SOURCES),
                       "summary": os.path.basename(args.out),
                       "hbm_read_bytes_per_dispatch": int(r["read_b"]),
                       "hbm_write_bytes_per_dispatch": int(r["write_b"]),
                       "hbm_bytes_per_dispatch": int(r["read_b"] + r["write_b"])}, f, indent=1)
            f.write("\n")
    print("\n".join(lines))


def write_stats(args) -> None:
    """Average duration of every kernel of a profile run (rocprofv3 --stats
    kernel_stats.csv), with the algorithmic bytes the run logged and the
    rate they imply."""
    if not args.out:
        raise SystemExit("--write-stats needs --out")
    algo = {"workload": args.title or "see the command", "classes": {},
            "definition": "not given for this run (see the bench line for the step's bytes)"}
    if args.algo:
        with open(args.algo) as f:
            algo = json.load(f)
    rows = []
    with open(args.write_stats, newline="") as f:
        for row in csv.DictReader(f):
            name = short_name(row["Name"])
            cls = kernel_class(name)
            if cls is None or cls == "calib":
                continue
            avg_us = float(row["AverageNs"]) / 1e3
            a = algo["classes"].get(cls, {})
            byts = (a.get("read") or 0) + (a.get("write") or 0)
            rows.append((name, int(row["Calls"]), avg_us, float(row["MinNs"]) / 1e3,
                         float(row["MaxNs"]) / 1e3, byts))
    lines = [f"# {args.title}" if args.title else "# rocprofv3 kernel stats",
             "# commands (repository root on the machine with the GPU, TMPDIR=/tmp):"]
    lines += [f"#   {c}" for c in args.cmd]
    lines += [f"# summary: python3 bench.py --write-stats <kernel_stats.csv> "
              f"{'--algo <algo json> ' if args.algo else ''}--out {os.path.basename(args.out)}",
              f"# source digest (code of {', '.join(ALL_SOURCES)}): {src_digest(*ALL_SOURCES)}",
              "", f"Workload: {algo['workload']}.",
              "Distinct experts per expert call (mean): " + (", ".join(
                  f"{kd} {sum(v) / len(v):.2f} over {len(v)} calls"
                  for kd, v in algo.get("distinct_experts", {}).items()) or "none") + ".",
              "Algorithmic bytes per call (mean): " + algo["definition"], "",
              "| kernel | calls | avg us | min us | max us | algorithmic MB | TB/s | % of 8 TB/s |",
              "|---|---|---|---|---|---|---|---|"]
    for name, calls, avg, mn, mx, byts in rows:
        rate = byts / (avg * 1e-6) / 1e12 if byts else None
        lines.append(f"| {name} | {calls} | {avg:.2f} | {mn:.2f} | {mx:.2f} | "
                     f"{byts / 1e6:.1f} | " + (f"{rate:.2f} | {rate / 8:.1%} |" if rate else "— | — |"))
    path = os.path.join(PROFILES, os.path.basename(args.out))
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def load_traffic(digest: str):
    """HBM bytes per lm_head dispatch from committed rocprofv3 counter runs,
    or None when they are missing or were taken on different kernel source."""
    path = os.path.join(PROFILES, "lmhead_argmax_counters.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        c = json.load(f)
    if c.get("source_digest") != digest:
        return None
    return c.get("hbm_bytes_per_dispatch")


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


# ------------------------------------------------------------------- bench

def main():
    args = parse()
    if args.write_counters:
        write_counters(args)
        return
    if args.write_stats:
        write_stats(args)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the multi-GPU sharding is a design note, not built)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import moe_speculative_verify_amd as mv
    import synth

    assert torch.cuda.is_available(), "bench needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    L = mv.lib()

    cfg = synth.WORKLOADS["layer_m6"]
    H, E, I, k = cfg["H"], cfg["E"], cfg["I"], cfg["k"]
    V = synth.WORKLOADS["lmhead"]["V"]
    M = args.M
    profiling = args.profile_steps > 0

    # ------------------------------------------------------------ weights
    t0 = time.time()
    K_ = synth.KIND
    layers = []
    for l in range(args.layers):
        layers.append(dict(
            router=synth.device_normal_bf16((E, H), synth.WEIGHT_STD, synth.WEIGHT_SEED, l, K_["router"]),
            gate=synth.device_normal_bf16((E, I, H), synth.WEIGHT_STD, synth.WEIGHT_SEED, l, K_["gate"]),
            up=synth.device_normal_bf16((E, I, H), synth.WEIGHT_STD, synth.WEIGHT_SEED, l, K_["up"]),
            down=synth.device_normal_bf16((E, H, I), synth.WEIGHT_STD, synth.WEIGHT_SEED, l, K_["down"]),
            # one shared expert per layer (the shared-expert variant's extra bucket)
            s_gate=synth.device_normal_bf16((I, H), synth.WEIGHT_STD, synth.WEIGHT_SEED, l, 50 + K_["gate"]),
            s_up=synth.device_normal_bf16((I, H), synth.WEIGHT_STD, synth.WEIGHT_SEED, l, 50 + K_["up"]),
            s_down=synth.device_normal_bf16((H, I), synth.WEIGHT_STD, synth.WEIGHT_SEED, l, 50 + K_["down"]),
        ))
        log(f"layer {l} weights generated ({time.time() - t0:.1f} s)")
    lms = [synth.device_normal_bf16((V, H), synth.WEIGHT_STD, synth.WEIGHT_SEED, 100 + c,
                                    K_["lm_head"]) for c in range(args.lm_copies)]
    routers = [synth.device_normal_bf16((E, H), synth.WEIGHT_STD, synth.WEIGHT_SEED, 200 + c,
                                        K_["router"]) for c in range(args.router_copies)]
    # fp8 experts (E4M3 codes + fp32 row scales) for the fp8 lines; the router
    # stays bf16 (each rotated layer's own); two fp8 lm_head copies
    layers8 = []
    for l in range(args.fp8_layers if not profiling else min(2, args.fp8_layers)):
        qg, sg = synth.device_fp8_rows((E, I, H), synth.WEIGHT_STD, synth.WEIGHT_SEED, 300 + l, K_["gate"])
        qu, su = synth.device_fp8_rows((E, I, H), synth.WEIGHT_STD, synth.WEIGHT_SEED, 300 + l, K_["up"])
        qd, sd = synth.device_fp8_rows((E, H, I), synth.WEIGHT_STD, synth.WEIGHT_SEED, 300 + l, K_["down"])
        layers8.append(dict(router=layers[l % len(layers)]["router"], gate=qg, s_gate=sg, up=qu,
                            s_up=su, down=qd, s_down=sd))
    lms8 = [synth.device_fp8_rows((V, H), synth.WEIGHT_STD, synth.WEIGHT_SEED, 400 + c,
                                  K_["lm_head"]) for c in range(2 if layers8 else 0)]
    log(f"weights ready: {torch.cuda.memory_allocated() / 1e9:.1f} GB ({time.time() - t0:.1f} s)")

    def up(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)

    def check(fn, st):
        if st != 0:
            raise RuntimeError(f"{fn}: {mv.status_str(st)}")

    eps = ctypes.c_float(1e-6)
    gain = up(synth.norm_gain(H))
    per_expert = 3 * I * H * 2
    per_expert8 = 3 * I * H + (2 * I + H) * 4          # fp8 codes + row scales

    class Layer:
        """One verify width's inputs, outputs and workspace, and the raw
        C-ABI argument tuples of one layer entry point over the rotating
        layers (built once, so timed loops only enqueue)."""

        def __init__(self, Ms, alpha, kind="bf16", identical=False, tag=None):
            self.M, self.alpha, self.kind = Ms, alpha, kind
            xs = synth.activations(Ms, H, seed=synth.ACT_SEED, tag=10 + Ms if tag is None else tag)
            if identical:
                xs = np.repeat(xs[:1], Ms, axis=0)
            self.x = up(xs)
            self.bias = None if alpha is None else torch.from_numpy(synth.zipf_bias(E, alpha)).to(dev)
            self.idx = torch.empty((Ms, k), dtype=torch.int32, device=dev)
            self.tw = torch.empty((Ms, k), dtype=torch.float32, device=dev)
            self.out = torch.empty((Ms, H), dtype=torch.float32, device=dev)
            self.ws = torch.zeros(L.moe_layer_workspace_bytes(Ms, H, I, E, k), dtype=torch.uint8,
                                  device=dev)
            if kind == "norm":
                self.hn = up(synth.hidden_states(Ms, H, tag=10 + Ms))
                self.xn = torch.empty((Ms, H), dtype=torch.bfloat16, device=dev)
            self.fn = {"bf16": L.moe_layer, "fp8": L.moe_layer_fp8, "norm": L.moe_layer_rmsnorm,
                       "shared": L.moe_layer_shared}[kind]
            self.weights = layers8 if kind == "fp8" else layers
            self.n = len(self.weights)
            self.D = None

        def args(self, l, stream):
            Lw = self.weights[l % self.n]
            b = self.bias.data_ptr() if self.bias is not None else None
            tail = (self.M, H, I, E, k)
            outs = (self.idx.data_ptr(), self.tw.data_ptr(), self.out.data_ptr(),
                    self.ws.data_ptr(), self.ws.numel(), stream)
            if self.kind == "bf16":
                return (self.x.data_ptr(), Lw["router"].data_ptr(), b, Lw["gate"].data_ptr(),
                        Lw["up"].data_ptr(), Lw["down"].data_ptr()) + tail + outs
            if self.kind == "fp8":
                return (self.x.data_ptr(), Lw["router"].data_ptr(), b, Lw["gate"].data_ptr(),
                        Lw["s_gate"].data_ptr(), Lw["up"].data_ptr(), Lw["s_up"].data_ptr(),
                        Lw["down"].data_ptr(), Lw["s_down"].data_ptr()) + tail + outs
            if self.kind == "shared":
                return (self.x.data_ptr(), Lw["router"].data_ptr(), b, Lw["gate"].data_ptr(),
                        Lw["up"].data_ptr(), Lw["down"].data_ptr(), Lw["s_gate"].data_ptr(),
                        Lw["s_up"].data_ptr(), Lw["s_down"].data_ptr()) + tail + outs
            return (self.hn.data_ptr(), gain.data_ptr(), eps, Lw["router"].data_ptr(), b,
                    Lw["gate"].data_ptr(), Lw["up"].data_ptr(), Lw["down"].data_ptr()) + tail + (
                    self.xn.data_ptr(),) + outs

        def call(self, l, stream):
            check(self.fn.__name__, self.fn(*self.args(l, stream)))

        def routing(self, stream):
            """Distinct experts each rotating layer selects (a pass over them)."""
            D = []
            for l in range(self.n):
                self.call(l, stream)
                torch.cuda.synchronize()
                D.append(len(np.unique(self.idx.cpu().numpy())))
            self.D = D
            return D

        def bytes(self, l):
            """Algorithmic bytes of the call on rotating layer l."""
            pe = per_expert8 if self.kind == "fp8" else per_expert
            Ms = self.M
            io = Ms * H * 2 + Ms * k * 8 + Ms * H * 4 + (E * 4 if self.bias is not None else 0)
            if self.kind == "norm":       # the pre-norm rows and the gain in, the normalised rows out
                io += H * 2 + Ms * H * 2
            extra = 1 if self.kind == "shared" else 0
            return E * H * 2 + (self.D[l % self.n] + extra) * pe + io

    stream = torch.cuda.current_stream().cuda_stream
    h = up(synth.activations(M, H, tag=1))
    am = torch.empty(M, dtype=torch.int32, device=dev)
    # the verify chain (root, then M - 1 drafted candidates): seeded tokens;
    # the verdict's cost does not depend on how many are accepted
    chain = torch.from_numpy(np.random.default_rng(3).integers(0, V, size=M).astype(np.int32)).to(dev)
    acc = torch.empty(2, dtype=torch.int32, device=dev)
    ws_lm = torch.zeros(L.lmhead_argmax_workspace_bytes(M, V), dtype=torch.uint8, device=dev)
    ws_route = torch.zeros(L.moe_route_workspace_bytes(M, E), dtype=torch.uint8, device=dev)

    def lm_args(c, st):
        return (h.data_ptr(), lms[c % len(lms)].data_ptr(), chain.data_ptr(), M, H, V,
                am.data_ptr(), None, acc.data_ptr(), ws_lm.data_ptr(), ws_lm.numel(), st)

    # the same call as its two phases, so that events can bracket the GEMV
    # kernel alone (the roofline's kernel)
    def lm_keys_args(c, st):
        return (h.data_ptr(), lms[c % len(lms)].data_ptr(), M, H, V, ws_lm.data_ptr(),
                ws_lm.numel(), st)

    def lm_merge_args(st):
        return (M, V, am.data_ptr(), None, chain.data_ptr(), acc.data_ptr(), ws_lm.data_ptr(),
                ws_lm.numel(), st)

    def lm8_args(c, st):
        q, sc = lms8[c % len(lms8)]
        return (h.data_ptr(), q.data_ptr(), sc.data_ptr(), chain.data_ptr(), M, H, V,
                am.data_ptr(), None, acc.data_ptr(), ws_lm.data_ptr(), ws_lm.numel(), st)

    lm_bytes = V * H * 2 + M * H * 2 + M * 4 + M * 4 + 8
    lm8_bytes = V * H + V * 4 + M * H * 2 + M * 8 + 8

    main_layer = Layer(M, args.zipf_alpha, identical=args.identical_tokens, tag=0)
    route_idx = torch.empty((M, k), dtype=torch.int32, device=dev)
    route_tw = torch.empty((M, k), dtype=torch.float32, device=dev)
    xr = main_layer.x
    rbias = main_layer.bias
    route_args = [(xr.data_ptr(), r.data_ptr(), rbias.data_ptr() if rbias is not None else None,
                   M, H, E, k, route_idx.data_ptr(), route_tw.data_ptr(), None,
                   ws_route.data_ptr(), ws_route.numel(), stream) for r in routers]
    hn = up(synth.hidden_states(M, H))
    xnorm = torch.empty((M, H), dtype=torch.bfloat16, device=dev)
    rn_args = [(hn.data_ptr(), gain.data_ptr(), eps, r.data_ptr(),
                rbias.data_ptr() if rbias is not None else None, M, H, E, k, xnorm.data_ptr(),
                route_idx.data_ptr(), route_tw.data_ptr(), None, ws_route.data_ptr(),
                ws_route.numel(), stream) for r in routers]
    route_bytes = E * H * 2 + M * H * 2 + M * k * 8 + (E * 4 if rbias is not None else 0)

    if profiling:
        profile(args, locals())
        return

    # ------------------------------------------- timed steps (events per call)
    D = main_layer.routing(stream)
    nl = main_layer.n
    K = args.steps
    for s in range(args.warmup):
        main_layer.call(s, stream)
        check("lmhead_greedy_verify", L.lmhead_greedy_verify(*lm_args(s, stream)))
    torch.cuda.synchronize()
    # the lm_head as its two phases (what lmhead_greedy_verify enqueues, bitwise
    # the same outputs), with an event between them: the GEMV kernel's own time
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(K)]
    t_start = time.perf_counter()
    for i, s in enumerate(range(args.warmup, args.warmup + K)):
        evs[i][0].record()
        main_layer.call(s, stream)
        evs[i][1].record()
        check("lmhead_partial_keys", L.lmhead_partial_keys(*lm_keys_args(s, stream)))
        evs[i][2].record()
        check("lmhead_merge_keys", L.lmhead_merge_keys(*lm_merge_args(stream)))
        evs[i][3].record()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t_start) * 1e3 / K
    gpu_ms = evs[0][0].elapsed_time(evs[K - 1][3]) / K
    layer_us = [evs[i][0].elapsed_time(evs[i][1]) * 1e3 for i in range(K)]
    lm_us = [evs[i][1].elapsed_time(evs[i][3]) * 1e3 for i in range(K)]
    lm_gemv_us = [evs[i][1].elapsed_time(evs[i][2]) * 1e3 for i in range(K)]
    layer_us_mean = sum(layer_us) / K
    lm_us_mean = sum(lm_us) / K
    lm_gemv_us_mean = sum(lm_gemv_us) / K
    # the roofline kernel's average launch duration: RB back-to-back GEMV
    # launches alternating the two lm_head copies (each cold: the other's
    # 805 MB were read in between), bracketed by one pair of events, so that
    # each launch's dispatch latency hides behind the kernel before it
    RB = 16
    rb_ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    rb_ev[0].record()
    for j in range(RB):
        check("lmhead_partial_keys", L.lmhead_partial_keys(*lm_keys_args(j, stream)))
    rb_ev[1].record()
    torch.cuda.synchronize()
    lm_gemv_b2b_us = rb_ev[0].elapsed_time(rb_ev[1]) * 1e3 / RB
    lm_gemv_gbps = lm_bytes / (lm_gemv_b2b_us * 1e-6) / 1e9
    layer_bytes_mean = sum(main_layer.bytes(s) for s in range(args.warmup, args.warmup + K)) / K
    layer_gbps = layer_bytes_mean / (layer_us_mean * 1e-6) / 1e9
    lm_gbps = lm_bytes / (lm_us_mean * 1e-6) / 1e9
    log(f"{K} steps: {wall_ms * 1e3:.1f} us/step wall, {gpu_ms * 1e3:.1f} us/step events; "
        f"layer {layer_us_mean:.2f} us ({layer_gbps / HBM_PEAK_GBPS:.1%}), "
        f"lm_head {lm_us_mean:.2f} us ({lm_gbps / HBM_PEAK_GBPS:.1%}; GEMV {lm_gemv_us_mean:.2f} us)")
    eager_out = (main_layer.idx.clone(), main_layer.tw.clone(), main_layer.out.clone(),
                 am.clone(), acc.clone())
    last = args.warmup + K - 1

    # -------------------- graph: N steps captured once, replayed, timed by events
    graph = None
    if args.graph_steps > 0:
        G = args.graph_steps
        cap = torch.cuda.Stream()
        g_step = torch.cuda.CUDAGraph()
        g_layer = torch.cuda.CUDAGraph()
        # steps last - G + 1 .. last, so the last replayed step is the last eager one
        first = last - G + 1
        with torch.cuda.graph(g_step, stream=cap):
            st = cap.cuda_stream
            for s in range(first, last + 1):
                main_layer.call(s, st)
                check("lmhead_greedy_verify", L.lmhead_greedy_verify(*lm_args(s, st)))
        with torch.cuda.graph(g_layer, stream=cap):
            st = cap.cuda_stream
            for s in range(first, last + 1):
                main_layer.call(s, st)
        reps = 4
        g_step.replay()
        torch.cuda.synchronize()
        same = all(torch.equal(a, b) for a, b in zip(
            eager_out, (main_layer.idx, main_layer.tw, main_layer.out, am, acc)))
        ge = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
        ge[0].record()
        for r in range(reps):
            g_step.replay()
            ge[r + 1].record()
        torch.cuda.synchronize()
        step_us_g = sum(ge[r].elapsed_time(ge[r + 1]) for r in range(reps)) * 1e3 / (reps * G)
        g_layer.replay()
        torch.cuda.synchronize()
        ge[0].record()
        for r in range(reps):
            g_layer.replay()
            ge[r + 1].record()
        torch.cuda.synchronize()
        layer_us_g = sum(ge[r].elapsed_time(ge[r + 1]) for r in range(reps)) * 1e3 / (reps * G)
        gbytes = sum(main_layer.bytes(s) for s in range(first, last + 1)) / G
        graph = {"steps_per_graph": G, "replays": reps,
                 "step_us": round(step_us_g, 2),
                 "moe_layer_us": round(layer_us_g, 2),
                 "moe_layer_GBps": round(gbytes / (layer_us_g * 1e-6) / 1e9, 1),
                 "moe_layer_frac": round(gbytes / (layer_us_g * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
                 "replay_equals_eager": same,
                 "timing": "HIP events on the replay stream around each replay of a graph "
                           "holding N captured steps (moe_layer + lmhead_greedy_verify, or the "
                           "layer alone), divided by N"}
        log(f"graph of {G} steps: step {step_us_g:.2f} us, layer {layer_us_g:.2f} us, "
            f"replay equals eager: {same}")
        del g_step, g_layer

    # ----------------------------------------- gate only, rotating router copies
    R = len(route_args)
    for s in range(min(R, 16)):
        check("moe_route", L.moe_route(*route_args[s]))
    torch.cuda.synchronize()
    re0 = torch.cuda.Event(enable_timing=True)
    re1 = torch.cuda.Event(enable_timing=True)
    re0.record()
    for s in range(R):
        check("moe_route", L.moe_route(*route_args[s]))
    re1.record()
    torch.cuda.synchronize()
    route_us = re0.elapsed_time(re1) * 1e3 / R

    # gate coldness: the same calls cycling over fewer distinct copies (the
    # time rises to a plateau once the copies no longer fit the caches)
    gate_sweep = {}
    for n in sorted({min(c, R) for c in (1, 8, 32, 128, R)}):
        for s in range(n):
            check("moe_route", L.moe_route(*route_args[s]))
        torch.cuda.synchronize()
        re0.record()
        for s in range(2 * R):
            check("moe_route", L.moe_route(*route_args[s % n]))
        re1.record()
        torch.cuda.synchronize()
        gate_sweep[str(n)] = round(re0.elapsed_time(re1) * 1e3 / (2 * R), 2)

    # the gate as a steady stream: 128 back-to-back calls on distinct cold
    # copies captured in one HIP graph, replayed, timed by events / 128
    gate_graph = None
    if args.graph_steps > 0:
        GN = min(128, R)
        capg = torch.cuda.Stream()
        g_gate = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g_gate, stream=capg):
            for s in range(GN):
                check("moe_route", L.moe_route(*(route_args[s][:-1] + (capg.cuda_stream,))))
        g_gate.replay()
        torch.cuda.synchronize()
        reps = 4
        ge = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
        ge[0].record()
        for r in range(reps):
            g_gate.replay()
            ge[r + 1].record()
        torch.cuda.synchronize()
        gate_graph_us = sum(ge[r].elapsed_time(ge[r + 1]) for r in range(reps)) * 1e3 / (reps * GN)
        gate_graph = {"calls_per_graph": GN, "replays": reps, "us": round(gate_graph_us, 2),
                      "GBps": round(route_bytes / (gate_graph_us * 1e-6) / 1e9, 1)}
        del g_gate
        log(f"gate graph: {GN} back-to-back calls, {gate_graph_us:.2f} us per call "
            f"({gate_graph['GBps']} GB/s)")

    for s in range(min(R, 16)):
        check("moe_route_rmsnorm", L.moe_route_rmsnorm(*rn_args[s]))
    torch.cuda.synchronize()
    re0.record()
    for s in range(R):
        check("moe_route_rmsnorm", L.moe_route_rmsnorm(*rn_args[s]))
    re1.record()
    torch.cuda.synchronize()
    route_norm_us = re0.elapsed_time(re1) * 1e3 / R

    # the measured HBM read ceiling: a plain streaming read (grid-stride
    # non-temporal 16-byte loads) over 4 rotating 1 GiB buffers
    probe_bufs = [torch.empty(2**30, dtype=torch.uint8, device=dev) for _ in range(4)]
    for b_ in probe_bufs:
        b_.fill_(1)
    sums = torch.empty(mv.HBM_PROBE_GROUPS, dtype=torch.int32, device=dev)
    for b_ in probe_bufs[:2]:
        mv.moe_hbm_read_probe(b_, sums)
    torch.cuda.synchronize()
    re0.record()
    for s in range(16):
        mv.moe_hbm_read_probe(probe_bufs[s % 4], sums)
    re1.record()
    torch.cuda.synchronize()
    probe_gbps = 16 * 2**30 / (re0.elapsed_time(re1) * 1e-3) / 1e9
    del probe_bufs
    log(f"streaming-read probe: {probe_gbps:.0f} GB/s")

    # ------------------------------------------- layer at other widths / kinds
    def timed(lay, steps=32, warm=8, n=None):
        """Mean per-call us and algorithmic GB/s of `lay` over its rotating
        layers (or the first n of them), every call bracketed by events."""
        n = lay.n if n is None else n
        if lay.D is None:
            lay.routing(stream)
        for s in range(warm):
            lay.call(s % n, stream)
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        for i in range(steps):
            ev[i].record()
            lay.call((warm + i) % n, stream)
        ev[steps].record()
        torch.cuda.synchronize()
        us = sum(ev[i].elapsed_time(ev[i + 1]) for i in range(steps)) * 1e3 / steps
        byts = sum(lay.bytes((warm + i) % n) for i in range(steps)) / steps
        gbps = byts / (us * 1e-6) / 1e9
        return {"M": lay.M, "zipf_alpha": lay.alpha, "kind": lay.kind, "layers_rotated": n,
                "us": round(us, 2), "GBps": round(gbps, 1), "frac": round(gbps / HBM_PEAK_GBPS, 4),
                "bytes": int(byts), "distinct_experts_mean": round(sum(lay.D[:n]) / n, 2)}

    widths = [timed(Layer(m, a)) for m, a in ((1, None), (1, 1.0), (16, None), (16, 1.0))]
    log("layer widths: " + ", ".join(f"M={r['M']} alpha={r['zipf_alpha']}: {r['us']} us "
                                     f"({r['frac']:.1%})" for r in widths))
    # expert-layer coldness: the M = 6 (and M = 1) layer cycling over 1, 2, 4
    # and 16 distinct layers
    cold = {}
    for Ms in (1, M):
        lay = main_layer if Ms == M else Layer(1, args.zipf_alpha, tag=0)
        cold[f"M{Ms}"] = {str(n): timed(lay, n=n)["us"] for n in (1, 2, 4, min(16, lay.n))}
    log(f"layer coldness (us by layers rotated): {cold}")
    layer_norm = timed(Layer(M, args.zipf_alpha, kind="norm"))
    layer_shared = [timed(Layer(m, args.zipf_alpha, kind="shared")) for m in (1, M, 16)]
    log("layer with a shared expert: " + ", ".join(f"M={r['M']}: {r['us']} us ({r['frac']:.1%})"
                                                  for r in layer_shared))
    fp8 = None
    if layers8:
        l8 = [timed(Layer(m, a, kind="fp8")) for m, a in ((1, None), (M, args.zipf_alpha),
                                                          (16, None), (16, 1.0))]
        for s in range(4):
            check("lmhead_greedy_verify_fp8", L.lmhead_greedy_verify_fp8(*lm8_args(s, stream)))
        torch.cuda.synchronize()
        ev8 = [torch.cuda.Event(enable_timing=True) for _ in range(33)]
        for i in range(32):
            ev8[i].record()
            check("lmhead_greedy_verify_fp8", L.lmhead_greedy_verify_fp8(*lm8_args(i, stream)))
        ev8[32].record()
        torch.cuda.synchronize()
        lm8_us = sum(ev8[i].elapsed_time(ev8[i + 1]) for i in range(32)) * 1e3 / 32
        lm8_gbps = lm8_bytes / (lm8_us * 1e-6) / 1e9
        fp8 = {"moe_layer": l8,
               "lm_head": {"us": round(lm8_us, 2), "GBps": round(lm8_gbps, 1),
                           "frac": round(lm8_gbps / HBM_PEAK_GBPS, 4), "bytes": lm8_bytes}}
        log("fp8 layer: " + ", ".join(f"M={r['M']} alpha={r['zipf_alpha']}: {r['us']} us "
                                      f"({r['frac']:.1%})" for r in l8)
            + f"; lm_head {lm8_us:.1f} us ({lm8_gbps / HBM_PEAK_GBPS:.1%})")
    log(f"router chain with norm: gate {route_norm_us:.2f} us (without {route_us:.2f}); "
        f"layer M={M} {layer_norm['us']} us")

    traffic = load_traffic(src_digest(*LM_DIGEST_SOURCES))

    # ---------------------------------------------------- CPU oracle baseline
    cpu = None if args.no_cpu_baseline else cpu_baseline(args, locals())

    res = {
        "metric": "cold-weight HBM GB/s (% of peak) + µs per MoE-layer verify step, M=6",
        "value": round(layer_gbps, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(wall_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"moe_layer_verify_step_M{M}",
                   "M": M, "hidden": H, "experts": E, "intermediate": I, "top_k": k,
                   "layers_rotated": nl, "zipf_alpha": args.zipf_alpha,
                   "step": "moe_layer then lmhead_greedy_verify; value is the moe_layer part "
                           "(events around each call), ms_per_step the whole step (wall)",
                   "seeds": [synth.WEIGHT_SEED, synth.ACT_SEED]},
        "frac_of_hbm_peak": round(layer_gbps / HBM_PEAK_GBPS, 4),
        "moe_layer": {"us": round(layer_us_mean, 2), "GBps": round(layer_gbps, 1),
                      "frac": round(layer_gbps / HBM_PEAK_GBPS, 4),
                      "bytes": int(layer_bytes_mean), "distinct_experts_mean": sum(D) / len(D)},
        "lm_head": {"workload": f"lmhead_greedy_verify {V}x{H} bf16, M={M}, enqueued as its two"
                                " phases (lmhead_partial_keys, lmhead_merge_keys)",
                    "us": round(lm_us_mean, 2), "GBps": round(lm_gbps, 1),
                    "frac": round(lm_gbps / HBM_PEAK_GBPS, 4), "bytes": lm_bytes,
                    "gemv_us": round(lm_gemv_us_mean, 2), "gemv_us_back_to_back": round(lm_gemv_b2b_us, 2),
                    "copies": len(lms)},
        "step_us_events": round(gpu_ms * 1e3, 2),
        "graph": graph,
        "moe_layer_other_widths": widths,
        "moe_layer_coldness_us_by_layers_rotated": cold,
        "hbm_read_probe": {"GBps": round(probe_gbps, 1),
                           "frac": round(probe_gbps / HBM_PEAK_GBPS, 4),
                           "kernel": "moe_hbm_read_probe: grid-stride non-temporal 16-byte loads, "
                                     "256 x 256 threads, 8 in flight per thread",
                           "bytes_per_call": 2**30, "buffers_rotated": 4, "calls": 16},
        "router_gate_cold": {"us": round(route_us, 2),
                             "GBps": round(route_bytes / (route_us * 1e-6) / 1e9, 1),
                             "copies": R, "us_by_distinct_copies": gate_sweep,
                             "graph_of_back_to_back_calls": gate_graph},
        "router_chain_rmsnorm": {"gate_us": round(route_norm_us, 2),
                                 "moe_layer_rmsnorm": layer_norm},
        "moe_layer_shared_expert": layer_shared,
        "fp8_weights": fp8,
        "roofline": {"kernel": f"lmhead_kernel<false> ({V}x{H} bf16, M={M}), the step's longest"
                               " kernel (lmhead_partial_keys, the GEMV phase of"
                               f" lmhead_greedy_verify): {RB} back-to-back launches on the two"
                               " cold lm_head copies between two events,"
                               f" {lm_gemv_b2b_us:.2f} us per launch",
                     "bound": "hbm", "achieved": round(lm_gemv_gbps, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(lm_gemv_gbps / HBM_PEAK_GBPS, 4),
                     "traffic": traffic},
        "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)


def cpu_baseline(args, env):
    """The CPU oracle on one full M = 6 step (router, experts and combine of
    one layer, then the lm_head argmax), single-threaded and on all the
    host's cores, best of args.cpu_reps each. Weights are read back (the
    selected experts only) before the timed region."""
    import numpy as np
    import torch

    import oracle

    lay, lms, h = env["main_layer"], env["lms"], env["h"]
    dev = lay.x.device

    def host_bits(t):
        return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)

    xb, hb = host_bits(lay.x), host_bits(h)
    bias_np = None if lay.bias is None else lay.bias.cpu().numpy()
    Lw = lay.weights[0]
    wr = host_bits(Lw["router"])
    r = oracle.route(xb, wr, bias_np, env["k"])
    uniq, inv = np.unique(r["idx"], return_inverse=True)
    sel = torch.as_tensor(uniq, dtype=torch.long, device=dev)
    sub = {key: host_bits(Lw[key].index_select(0, sel)) for key in ("gate", "up", "down")}
    wl = host_bits(lms[0])
    ids = inv.reshape(r["idx"].shape).astype(np.int32)
    o = oracle.load()
    nproc = len(os.sched_getaffinity(0))
    V = wl.shape[0]
    runs = {}
    for threads in (1, nproc):
        used = o.set_threads(threads)
        # the single-threaded lm_head runs on the first V/8 rows (13 s of
        # work in full) and is scaled to V rows: its time is linear in V
        rows = V // 8 if used == 1 else V
        wl_s = wl[:rows]
        best = None
        for _ in range(args.cpu_reps):
            t1 = time.perf_counter()
            rr = oracle.route(xb, wr, bias_np, env["k"])
            oracle.expert_ffn(xb, ids, rr["w"], sub["gate"], sub["up"], sub["down"])
            t2 = time.perf_counter()
            oracle.lmhead(hb, wl_s)
            t3 = time.perf_counter()
            lm_t = (t3 - t2) * V / rows
            if best is None or (t2 - t1) + lm_t < best[0]:
                best = ((t2 - t1) + lm_t, t2 - t1, lm_t, rows)
        runs[used] = best
        log(f"cpu oracle, {used} threads: step {best[0] * 1e3:.0f} ms (layer {best[1] * 1e3:.0f}, "
            f"lm_head {best[2] * 1e3:.0f} from {rows} rows), best of {args.cpu_reps}")
    o.set_threads(nproc)
    layer_b = lay.bytes(0)
    model = cpu_model()

    def rec(threads):
        t, tl, tm, rows = runs[threads]
        return {"layer_GBps": round(layer_b / tl / 1e9, 3), "layer_ms": round(tl * 1e3, 1),
                "lm_head_ms": round(tm * 1e3, 1), "lm_head_rows_timed": rows,
                "step_ms": round(t * 1e3, 1), "threads": threads}

    top = max(runs)
    return {"value": round(layer_b / runs[top][1] / 1e9, 3), "unit": "GB/s", "cores": top,
            "kind": "oracle", "cpu_model": model, "best_of": args.cpu_reps,
            "sample": f"one M={lay.M} MoE layer step (route + selected experts + combine, "
                      f"{len(uniq)} distinct experts, rotating layer 0) and one lm_head argmax "
                      f"({V} rows; {V // 8} rows single-threaded, scaled) in fp64; value = the "
                      f"layer's algorithmic bytes / its time on all {top} threads",
            "single_thread": rec(1), "all_cores": rec(top)}


def profile(args, env):
    """Profile mode: a calibration kernel of known traffic, then
    args.profile_steps rounds of every entry point the bench times, for
    rocprofv3 (kernel stats or HBM counters). With --algo-out, the
    algorithmic bytes per call of every kernel class are written there."""
    import numpy as np
    import torch

    L, check, stream = env["L"], env["check"], env["stream"]
    H, E, I, k, M, V = (env[n] for n in ("H", "E", "I", "k", "M", "V"))
    lay = env["main_layer"]
    Layer = env["Layer"]
    # calibration kernel: an int32 bitwise_not that reads and writes
    # calib_mib MiB, run cold twice
    n = args.calib_mib * 2**20 // 4
    dev = lay.x.device
    src = torch.ones(n, dtype=torch.int32, device=dev)
    dst = torch.empty_like(src)
    flush = torch.empty(n, dtype=torch.int32, device=dev)
    for _ in range(2):
        flush.fill_(0)
        torch.bitwise_not(src, out=dst)
    torch.cuda.synchronize()
    del src, dst, flush
    lay8 = Layer(M, args.zipf_alpha, kind="fp8", identical=args.identical_tokens, tag=0) \
        if env["layers8"] else None
    ids, ids8 = [], []
    for s in range(args.profile_steps):
        lay.call(s, stream)
        ids.append(lay.idx.clone())
        check("lmhead_greedy_verify", L.lmhead_greedy_verify(*env["lm_args"](s, stream)))
        check("moe_route", L.moe_route(*env["route_args"][s % len(env["route_args"])]))
        check("moe_route_rmsnorm", L.moe_route_rmsnorm(*env["rn_args"][s % len(env["rn_args"])]))
        if lay8 is not None:
            lay8.call(s, stream)
            ids8.append(lay8.idx.clone())
        if env["lms8"]:
            check("lmhead_greedy_verify_fp8",
                  L.lmhead_greedy_verify_fp8(*env["lm8_args"](s, stream)))
    torch.cuda.synchronize()
    classes = {}
    dist = {}
    for name, lst, up_b, dn_b in (("bf16", ids, 2 * I * H * 2, H * I * 2),
                                  ("fp8", ids8, 2 * I * (H + 4), H * (I + 4))):
        if not lst:
            continue
        Dl = [len(np.unique(t.cpu().numpy())) for t in lst]
        dist[name] = Dl
        wd = sum(Dl) / len(Dl)
        classes[f"up_{name}"] = {"read": wd * up_b + M * H * 2, "write": M * k * I * 2 + M * k * 8}
        classes[f"down_{name}"] = {"read": wd * dn_b + M * k * I * 2 + M * k * 8,
                                   "write": M * H * 4}
        log(f"profile {name} expert calls: distinct experts {Dl}")
    bias_b = E * 4 if lay.bias is not None else 0
    classes["route_partials"] = {"read": E * H * 2 + M * H * 2 + bias_b, "write": None}
    classes["route"] = {"read": E * H * 2 + M * H * 2 + bias_b, "write": M * k * 8}
    classes["route_norm"] = {"read": E * H * 2 + M * H * 2 + H * 2 + bias_b,
                             "write": M * k * 8 + M * H * 2}
    classes["lm_bf16"] = {"read": V * H * 2 + M * H * 2 + M * 4, "write": M * 4 + 8}
    classes["lm_fp8"] = {"read": V * H + V * 4 + M * H * 2 + M * 4, "write": M * 4 + 8}
    algo = {"workload": f"M={M}{' (identical tokens)' if args.identical_tokens else ''}, "
                        f"{E} experts, H={H}, I={I}, top-{k}, zipf alpha {args.zipf_alpha}, "
                        f"{lay.n} rotating bf16 layers, {len(env['layers8'])} fp8 layers, "
                        f"lm_head {V}x{H}",
            "M": M, "identical_tokens": args.identical_tokens, "zipf_alpha": args.zipf_alpha,
            "distinct_experts": dist,
            "definition": "up: D*2*I*H weights (2 B bf16; fp8 1 B + a 4 B scale per row) + "
                          "M*H*2 x; writes M*k*I*2 activations + M*k*8 ids and weights. down: "
                          "D*H*I weights + M*k*I*2 activations + M*k*8 ids and weights; writes "
                          "M*H*4. route: E*H*2 gate + M*H*2 x (+ E*4 bias; with the norm + H*2 "
                          "gain and M*H*2 normalised rows out). lm_head: V*H weights + M*H*2 "
                          "hidden states (+ V*4 scales for fp8). D = distinct experts of the call.",
            "classes": classes}
    if args.algo_out:
        os.makedirs(os.path.dirname(os.path.abspath(args.algo_out)), exist_ok=True)
        with open(args.algo_out, "w") as f:
            json.dump(algo, f, indent=1)
    log(f"profile run: {args.profile_steps} steps done")


if __name__ == "__main__":
    main()
