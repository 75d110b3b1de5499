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

Prints ONE JSON line. `value` is algorithmic bytes per step / step time in
GB/s, where algorithmic bytes = every distinct selected expert's weights once,
the router gate, the lm_head, and the activations and outputs.
"""
from __future__ import annotations

import argparse
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
    ap.add_argument("--cpu-sample-steps", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--profile-steps", type=int, default=0,
                    help="only run this many steps (for rocprofv3), print nothing else")
    ap.add_argument("--calib-mib", type=int, default=1024,
                    help="profile mode: size of the int32 bitwise_not calibration kernel "
                         "(reads and writes this many MiB)")
    ap.add_argument("--write-counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="no GPU: turn two rocprofv3 --pmc counter_collection.csv files "
                         "(FETCH_SIZE run, WRITE_SIZE run) of the profile mode into "
                         "profiles/lmhead_argmax_counters.json")
    return ap.parse_args()


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


CALIB_KERNEL = "bitwise_not"     # substring of the calibration kernel's name
LM_KERNEL = "lmhead_kernel<false>"   # the bf16 lm_head (the roofline kernel)
LM8_KERNEL = "lmhead_kernel<true>"   # the fp8 lm_head


def counter_means(path: str, counter: str) -> dict:
    """Mean per-dispatch value of `counter` for the lm_head kernel and the
    calibration kernel in one rocprofv3 counter_collection.csv."""
    import csv
    vals = {LM_KERNEL: [], LM8_KERNEL: [], CALIB_KERNEL: []}
    with open(path, newline="") as f:
        for row in csv.DictReader(f):
            if row.get("Counter_Name") != counter:
                continue
            for key in vals:
                if key in row.get("Kernel_Name", ""):
                    vals[key].append(float(row["Counter_Value"]))
    for key in (LM_KERNEL, CALIB_KERNEL):
        if not vals[key]:
            raise SystemExit(f"{path}: no {counter} rows for a kernel named *{key}*")
    if not vals[LM8_KERNEL]:
        del vals[LM8_KERNEL]
    return {key: sum(v) / len(v) for key, v in vals.items()} | {
        "dispatches": {key: len(v) for key, v in vals.items()}}


def write_counters(fetch_csv: str, write_csv: str, calib_mib: int) -> None:
    """FETCH_SIZE and WRITE_SIZE (KiB per dispatch) of lmhead_argmax, each
    scaled by what the same counter reads for the calibration kernel, which
    reads and writes calib_mib MiB: HBM bytes = KiB * 1024 / factor."""
    fe = counter_means(fetch_csv, "FETCH_SIZE")
    wr = counter_means(write_csv, "WRITE_SIZE")
    calib_bytes = calib_mib * 2**20
    f_fac = fe[CALIB_KERNEL] * 1024 / calib_bytes
    w_fac = wr[CALIB_KERNEL] * 1024 / calib_bytes
    lm_read = fe[LM_KERNEL] * 1024 / f_fac
    lm_write = wr[LM_KERNEL] * 1024 / w_fac
    out = {
        "kernel": "lmhead_greedy_verify (lmhead_kernel), 157184x2560 bf16, M=6",
        "source_digest": src_digest("lmhead.hip", "common.h"),
        "fetch_kib_per_dispatch": round(fe[LM_KERNEL], 1),
        "write_kib_per_dispatch": round(wr[LM_KERNEL], 3),
        "calibration": {"kernel": f"torch int32 {CALIB_KERNEL}, {calib_mib} MiB in and out",
                        "fetch_kib": round(fe[CALIB_KERNEL], 1),
                        "write_kib": round(wr[CALIB_KERNEL], 1),
                        "fetch_factor": round(f_fac, 4), "write_factor": round(w_fac, 4)},
        "hbm_read_bytes_per_dispatch": int(lm_read),
        "hbm_write_bytes_per_dispatch": int(lm_write),
        "hbm_bytes_per_dispatch": int(lm_read + lm_write),
        "dispatches": {"fetch_run": fe["dispatches"], "write_run": wr["dispatches"]},
    }
    if LM8_KERNEL in fe and LM8_KERNEL in wr:
        # the fp8 lm_head of the same runs: algorithmic 157184*2560 codes +
        # 157184 scales + h + outputs
        r8, w8 = fe[LM8_KERNEL] * 1024 / f_fac, wr[LM8_KERNEL] * 1024 / w_fac
        out["fp8"] = {"kernel": "lmhead_greedy_verify_fp8 (lmhead_kernel<true>), 157184x2560 e4m3, M=6",
                      "fetch_kib_per_dispatch": round(fe[LM8_KERNEL], 1),
                      "write_kib_per_dispatch": round(wr[LM8_KERNEL], 3),
                      "hbm_read_bytes_per_dispatch": int(r8),
                      "hbm_write_bytes_per_dispatch": int(w8),
                      "hbm_bytes_per_dispatch": int(r8 + w8)}
    os.makedirs(PROFILES, exist_ok=True)
    path = os.path.join(PROFILES, "lmhead_argmax_counters.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    print(json.dumps(out))


def load_traffic(kernel: str, digest: str):
    """HBM bytes per dispatch from committed rocprofv3 counter runs, or None
    when they are missing or were taken on different kernel source."""
    path = os.path.join(PROFILES, f"{kernel}_counters.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        c = json.load(f)
    if c.get("source_digest") != digest:
        return None
    return c.get("hbm_bytes_per_dispatch")


def main():
    args = parse()
    if args.write_counters:
        write_counters(args.write_counters[0], args.write_counters[1], args.calib_mib)
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

    # ------------------------------------------------------------ inputs
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
    for l in range(args.fp8_layers if not args.profile_steps else min(2, args.fp8_layers)):
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

    x = up(synth.activations(M, H))
    h = up(synth.activations(M, H, tag=1))
    bias = None
    if args.zipf_alpha is not None:
        bias = torch.from_numpy(synth.zipf_bias(E, args.zipf_alpha)).to(dev)
    idx = torch.empty((M, k), dtype=torch.int32, device=dev)
    tw = torch.empty((M, k), dtype=torch.float32, device=dev)
    out = torch.empty((M, H), dtype=torch.float32, device=dev)
    am = torch.empty(M, dtype=torch.int32, device=dev)
    # the verify chain (root, then M - 1 drafted candidates): seeded tokens;
    # the verdict's cost does not depend on how many are accepted
    chain = torch.from_numpy(np.random.default_rng(3).integers(0, V, size=M).astype(np.int32)).to(dev)
    acc = torch.empty(2, dtype=torch.int32, device=dev)
    ws_layer = torch.zeros(L.moe_layer_workspace_bytes(M, H, I, E, k), dtype=torch.uint8, device=dev)
    ws_lm = torch.zeros(L.lmhead_argmax_workspace_bytes(M, V), dtype=torch.uint8, device=dev)
    ws_route = torch.zeros(L.moe_route_workspace_bytes(M, E), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream().cuda_stream

    # raw C-ABI argument tuples, built once so the timed loop only enqueues
    layer_args = [(x.data_ptr(), Lw["router"].data_ptr(), bias.data_ptr() if bias is not None else None,
                   Lw["gate"].data_ptr(), Lw["up"].data_ptr(), Lw["down"].data_ptr(),
                   M, H, I, E, k, idx.data_ptr(), tw.data_ptr(), out.data_ptr(),
                   ws_layer.data_ptr(), ws_layer.numel(), stream) for Lw in layers]
    lm_args = [(h.data_ptr(), w.data_ptr(), chain.data_ptr(), M, H, V, am.data_ptr(), None,
                acc.data_ptr(), ws_lm.data_ptr(), ws_lm.numel(), stream) for w in lms]
    route_args = [(x.data_ptr(), r.data_ptr(), bias.data_ptr() if bias is not None else None,
                   M, H, E, k, idx.data_ptr(), tw.data_ptr(), None, ws_route.data_ptr(),
                   ws_route.numel(), stream) for r in routers]

    # the router chain with its norm in front (moe_route_rmsnorm): the same
    # rotating router copies, hidden states before the norm and a gain
    hn = up(synth.hidden_states(M, H))
    gain = up(synth.norm_gain(H))
    xnorm = torch.empty((M, H), dtype=torch.bfloat16, device=dev)
    eps = ctypes.c_float(1e-6)
    rn_args = [(hn.data_ptr(), gain.data_ptr(), eps, r.data_ptr(),
                bias.data_ptr() if bias is not None else None, M, H, E, k, xnorm.data_ptr(),
                idx.data_ptr(), tw.data_ptr(), None, ws_route.data_ptr(), ws_route.numel(),
                stream) for r in routers]

    def check(fn, st):
        if st != 0:
            raise RuntimeError(f"{fn}: {mv.status_str(st)}")

    def step(s):
        check("moe_layer", L.moe_layer(*layer_args[s % len(layer_args)]))
        check("lmhead_greedy_verify", L.lmhead_greedy_verify(*lm_args[s % len(lm_args)]))

    if args.profile_steps:
        # calibration kernel of known traffic for the HBM counters: an int32
        # bitwise_not that reads and writes calib_mib MiB, run cold twice
        n = args.calib_mib * 2**20 // 4
        src = torch.ones(n, dtype=torch.int32, device=dev)
        dst = torch.empty_like(src)
        flush = torch.empty(n, dtype=torch.int32, device=dev)
        for _ in range(2):
            flush.fill_(0)
            torch.bitwise_not(src, out=dst)
        torch.cuda.synchronize()
        del src, dst, flush
        p8 = [(x.data_ptr(), Lw["router"].data_ptr(), None, Lw["gate"].data_ptr(),
               Lw["s_gate"].data_ptr(), Lw["up"].data_ptr(), Lw["s_up"].data_ptr(),
               Lw["down"].data_ptr(), Lw["s_down"].data_ptr(), M, H, I, E, k, idx.data_ptr(),
               tw.data_ptr(), out.data_ptr(), ws_layer.data_ptr(), ws_layer.numel(), stream)
              for Lw in layers8]
        pl8 = [(h.data_ptr(), q.data_ptr(), sc.data_ptr(), chain.data_ptr(), M, H, V,
                am.data_ptr(), None, acc.data_ptr(), ws_lm.data_ptr(), ws_lm.numel(), stream)
               for q, sc in lms8]
        # the routing of every expert call is kept, so the expert kernels'
        # counters can be set against their algorithmic bytes
        ids, ids8 = [], []
        for s in range(args.profile_steps):
            step(s)
            ids.append(idx.clone())
            check("moe_route", L.moe_route(*route_args[s % len(route_args)]))
            check("moe_route_rmsnorm", L.moe_route_rmsnorm(*rn_args[s % len(rn_args)]))
            if p8 and M <= 9:
                check("moe_layer_fp8", L.moe_layer_fp8(*p8[s % len(p8)]))
                ids8.append(idx.clone())
            if pl8:
                check("lmhead_greedy_verify_fp8", L.lmhead_greedy_verify_fp8(*pl8[s % len(pl8)]))
        torch.cuda.synchronize()
        for name, lst, up_b, dn_b in (
                ("bf16", ids, 2 * I * H * 2, H * I * 2),
                ("fp8", ids8, 2 * I * (H + 4), H * (I + 4))):
            if not lst:
                continue
            D = [len(np.unique(t.cpu().numpy())) for t in lst]
            wd = sum(D) / len(D)
            # reads: weights + x (or the activations) + routing; writes: act, out
            log(f"profile {name} expert calls: distinct experts {D}; algorithmic bytes per call, "
                f"mean: up read {wd * up_b + M * H * 2 + M * k * 4:.0f} write {M * k * I * 2}, "
                f"down read {wd * dn_b + M * k * I * 2 + M * k * 8:.0f} write {M * H * 4}")
        log(f"profile run: {args.profile_steps} steps done")
        return

    # --------------------------------------------- algorithmic bytes per step
    D = []
    for l in range(len(layers)):
        check("moe_layer", L.moe_layer(*layer_args[l]))
        torch.cuda.synchronize()
        D.append(len(np.unique(idx.cpu().numpy())))
    per_expert = 3 * I * H * 2
    per_expert8 = 3 * I * H + (2 * I + H) * 4          # fp8 codes + row scales
    io_layer = M * H * 2 + M * k * 8 + M * H * 4 + (E * 4 if bias is not None else 0)
    layer_bytes = [E * H * 2 + d * per_expert + io_layer for d in D]
    lm_bytes = V * H * 2 + M * H * 2 + M * 4 + M * 4 + 8
    route_bytes = E * H * 2 + M * H * 2 + M * k * 8 + (E * 4 if bias is not None else 0)
    nl = len(layers)
    K = args.steps
    step_bytes_mean = (sum(layer_bytes[s % nl] for s in range(args.warmup, args.warmup + K)) / K
                       + lm_bytes)

    # --------------------------------------------------------- timed steps
    # HIP events on the launch stream bracket every call inside the timed
    # region: per-call durations for the roofline come from the same run
    for s in range(args.warmup):
        step(s)
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    t_start = time.perf_counter()
    for i, s in enumerate(range(args.warmup, args.warmup + K)):
        evs[i][0].record()
        check("moe_layer", L.moe_layer(*layer_args[s % nl]))
        evs[i][1].record()
        check("lmhead_greedy_verify", L.lmhead_greedy_verify(*lm_args[s % len(lm_args)]))
        evs[i][2].record()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t_start) * 1e3 / K
    gpu_ms = evs[0][0].elapsed_time(evs[K - 1][2]) / K
    log(f"{K} steps: {wall_ms * 1e3:.1f} us/step wall, {gpu_ms * 1e3:.1f} us/step events")
    layer_us = [evs[i][0].elapsed_time(evs[i][1]) * 1e3 for i in range(K)]
    lm_us = [evs[i][1].elapsed_time(evs[i][2]) * 1e3 for i in range(K)]
    layer_us_mean = sum(layer_us) / K
    lm_us_mean = sum(lm_us) / K
    layer_bytes_mean = sum(layer_bytes[s % nl] for s in range(args.warmup, args.warmup + K)) / K

    # gate only: router GEMV + top-k over rotating router copies
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
    for n in sorted({min(c, R) for c in (8, 32, 128, R)}):
        for s in range(n):
            check("moe_route", L.moe_route(*route_args[s]))
        torch.cuda.synchronize()
        g0 = torch.cuda.Event(enable_timing=True)
        g1 = torch.cuda.Event(enable_timing=True)
        g0.record()
        for s in range(2 * R):
            check("moe_route", L.moe_route(*route_args[s % n]))
        g1.record()
        torch.cuda.synchronize()
        gate_sweep[str(n)] = round(g0.elapsed_time(g1) * 1e3 / (2 * R), 2)

    # the measured HBM read ceiling: a plain streaming read (grid-stride
    # non-temporal 16-byte loads) over 4 rotating 1 GiB buffers
    probe_bufs = [torch.empty(2**30, dtype=torch.uint8, device=dev) for _ in range(4)]
    for b_ in probe_bufs:
        b_.fill_(1)
    sums = torch.empty(mv.HBM_PROBE_GROUPS, dtype=torch.int32, device=dev)
    for b_ in probe_bufs[:2]:
        mv.moe_hbm_read_probe(b_, sums)
    torch.cuda.synchronize()
    p0 = torch.cuda.Event(enable_timing=True)
    p1 = torch.cuda.Event(enable_timing=True)
    p0.record()
    for s in range(16):
        mv.moe_hbm_read_probe(probe_bufs[s % 4], sums)
    p1.record()
    torch.cuda.synchronize()
    probe_gbps = 16 * 2**30 / (p0.elapsed_time(p1) * 1e-3) / 1e9
    del probe_bufs
    log(f"streaming-read probe: {probe_gbps:.0f} GB/s")

    for s in range(min(R, 16)):
        check("moe_route_rmsnorm", L.moe_route_rmsnorm(*rn_args[s]))
    torch.cuda.synchronize()
    re0.record()
    for s in range(R):
        check("moe_route_rmsnorm", L.moe_route_rmsnorm(*rn_args[s]))
    re1.record()
    torch.cuda.synchronize()
    route_norm_us = re0.elapsed_time(re1) * 1e3 / R

    # layer step at the other verify widths of the workload, uniform and
    # Zipf-biased routing (same 16 rotating layers, cold); with norm=True the
    # router chain's norm runs in front (moe_layer_rmsnorm)
    def layer_at(Ms, alpha, steps=32, warm=8, norm=False, shared=False, fp8=False):
        xs = up(synth.activations(Ms, H, seed=synth.ACT_SEED, tag=10 + Ms))
        bs = None if alpha is None else torch.from_numpy(synth.zipf_bias(E, alpha)).to(dev)
        ids = torch.empty((Ms, k), dtype=torch.int32, device=dev)
        tws = torch.empty((Ms, k), dtype=torch.float32, device=dev)
        outs = torch.empty((Ms, H), dtype=torch.float32, device=dev)
        ws = torch.zeros(L.moe_layer_workspace_bytes(Ms, H, I, E, k), dtype=torch.uint8, device=dev)
        if norm:
            hs = up(synth.hidden_states(Ms, H, tag=10 + Ms))
            xns = torch.empty((Ms, H), dtype=torch.bfloat16, device=dev)
            a = [(hs.data_ptr(), gain.data_ptr(), eps, Lw["router"].data_ptr(),
                  bs.data_ptr() if bs is not None else None,
                  Lw["gate"].data_ptr(), Lw["up"].data_ptr(), Lw["down"].data_ptr(),
                  Ms, H, I, E, k, xns.data_ptr(), ids.data_ptr(), tws.data_ptr(),
                  outs.data_ptr(), ws.data_ptr(), ws.numel(), stream) for Lw in layers]
            fn = L.moe_layer_rmsnorm
        elif fp8:
            a = [(xs.data_ptr(), Lw["router"].data_ptr(), bs.data_ptr() if bs is not None else None,
                  Lw["gate"].data_ptr(), Lw["s_gate"].data_ptr(), Lw["up"].data_ptr(),
                  Lw["s_up"].data_ptr(), Lw["down"].data_ptr(), Lw["s_down"].data_ptr(),
                  Ms, H, I, E, k, ids.data_ptr(), tws.data_ptr(), outs.data_ptr(),
                  ws.data_ptr(), ws.numel(), stream) for Lw in layers8]
            fn = L.moe_layer_fp8
        elif shared:
            a = [(xs.data_ptr(), Lw["router"].data_ptr(), bs.data_ptr() if bs is not None else None,
                  Lw["gate"].data_ptr(), Lw["up"].data_ptr(), Lw["down"].data_ptr(),
                  Lw["s_gate"].data_ptr(), Lw["s_up"].data_ptr(), Lw["s_down"].data_ptr(),
                  Ms, H, I, E, k, ids.data_ptr(), tws.data_ptr(), outs.data_ptr(),
                  ws.data_ptr(), ws.numel(), stream) for Lw in layers]
            fn = L.moe_layer_shared
        else:
            a = [(xs.data_ptr(), Lw["router"].data_ptr(), bs.data_ptr() if bs is not None else None,
                  Lw["gate"].data_ptr(), Lw["up"].data_ptr(), Lw["down"].data_ptr(),
                  Ms, H, I, E, k, ids.data_ptr(), tws.data_ptr(), outs.data_ptr(),
                  ws.data_ptr(), ws.numel(), stream) for Lw in layers]
            fn = L.moe_layer
        Ds = []
        nla = len(a)
        for l in range(nla):
            check("moe_layer", fn(*a[l]))
            torch.cuda.synchronize()
            Ds.append(len(np.unique(ids.cpu().numpy())))
        # with the norm: the pre-norm rows and the gain in, the normalised rows out
        io = (Ms * H * 2 + Ms * k * 8 + Ms * H * 4 + (E * 4 if bs is not None else 0)
              + (H * 2 + Ms * H * 2 if norm else 0))
        for s in range(warm):
            check("moe_layer", fn(*a[s % nla]))
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        for i in range(steps):
            ev[i].record()
            check("moe_layer", fn(*a[(warm + i) % nla]))
        ev[steps].record()
        torch.cuda.synchronize()
        us = sum(ev[i].elapsed_time(ev[i + 1]) for i in range(steps)) * 1e3 / steps
        pe = per_expert8 if fp8 else per_expert
        byts = sum(E * H * 2 + (Ds[(warm + i) % nla] + (1 if shared else 0)) * pe + io
                   for i in range(steps)) / steps
        gbps = byts / (us * 1e-6) / 1e9
        return {"M": Ms, "zipf_alpha": alpha, "rmsnorm": norm, "shared_expert": shared,
                "fp8_experts": fp8,
                "us": round(us, 2),
                "GBps": round(gbps, 1),
                "frac": round(gbps / HBM_PEAK_GBPS, 4), "bytes": int(byts),
                "distinct_experts_mean": sum(Ds) / len(Ds)}

    layer_sweep = [layer_at(m, a) for m, a in ((1, None), (1, 1.0), (16, None), (16, 1.0))]
    layer_norm = layer_at(M, args.zipf_alpha, norm=True)
    layer_shared = [layer_at(m, args.zipf_alpha, shared=True) for m in (1, M, 16)]
    fp8 = None
    if layers8:
        # fp8 experts at M = 1 and the step's M (the activations of M*k pairs
        # must fit in LDS: M <= 9 at I = 1024, k = 8), and the fp8 lm_head
        # with the verdict, cold over two copies
        l8 = [layer_at(m, args.zipf_alpha, fp8=True) for m in (1, M)]
        lm8_args = [(h.data_ptr(), q.data_ptr(), sc.data_ptr(), chain.data_ptr(), M, H, V,
                     am.data_ptr(), None, acc.data_ptr(), ws_lm.data_ptr(), ws_lm.numel(), stream)
                    for q, sc in lms8]
        for s in range(4):
            check("lmhead_greedy_verify_fp8", L.lmhead_greedy_verify_fp8(*lm8_args[s % 2]))
        torch.cuda.synchronize()
        ev8 = [torch.cuda.Event(enable_timing=True) for _ in range(33)]
        for i in range(32):
            ev8[i].record()
            check("lmhead_greedy_verify_fp8", L.lmhead_greedy_verify_fp8(*lm8_args[i % 2]))
        ev8[32].record()
        torch.cuda.synchronize()
        lm8_us = sum(ev8[i].elapsed_time(ev8[i + 1]) for i in range(32)) * 1e3 / 32
        lm8_bytes = V * H + V * 4 + M * H * 2 + M * 8 + 8
        lm8_gbps = lm8_bytes / (lm8_us * 1e-6) / 1e9
        fp8 = {"moe_layer": l8,
               "lm_head": {"us": round(lm8_us, 2), "GBps": round(lm8_gbps, 1),
                           "frac": round(lm8_gbps / HBM_PEAK_GBPS, 4), "bytes": lm8_bytes},
               "step_us_M": round(l8[-1]["us"] + lm8_us, 2)}
        log(f"fp8: layer M=1 {l8[0]['us']} us ({l8[0]['frac']:.1%}), M={M} {l8[1]['us']} us "
            f"({l8[1]['frac']:.1%}); lm_head {lm8_us:.1f} us ({lm8_gbps / HBM_PEAK_GBPS:.1%})")
    log("layer with a shared expert: " + ", ".join(f"M={r['M']}: {r['us']} us ({r['frac']:.1%})"
                                                  for r in layer_shared))
    log(f"router chain with norm: gate {route_norm_us:.2f} us (without {route_us:.2f}); "
        f"layer M={M} {layer_norm['us']} us")
    log("layer sweep: " + ", ".join(f"M={r['M']} alpha={r['zipf_alpha']}: {r['us']} us "
                                    f"({r['frac']:.1%})" for r in layer_sweep))

    lm_gbps = lm_bytes / (lm_us_mean * 1e-6) / 1e9
    layer_gbps = layer_bytes_mean / (layer_us_mean * 1e-6) / 1e9
    traffic = load_traffic("lmhead_argmax", src_digest("lmhead.hip", "common.h"))

    # ------------------------------------------------- CPU oracle baseline
    cpu = None
    if not args.no_cpu_baseline and args.cpu_sample_steps > 0:
        import oracle

        def host_bits(t):
            return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)

        n = args.cpu_sample_steps
        xb, hb = host_bits(x), host_bits(h)
        bias_np = None if bias is None else bias.cpu().numpy()
        samples = []
        for s in range(n):
            Lw = layers[s % nl]
            wr = host_bits(Lw["router"])
            # routing first (untimed) to know which experts to read back
            r = oracle.route(xb, wr, bias_np, k)
            uniq, inv = np.unique(r["idx"], return_inverse=True)
            sel = torch.as_tensor(uniq, dtype=torch.long, device=dev)
            sub = {key: host_bits(Lw[key].index_select(0, sel)) for key in ("gate", "up", "down")}
            wl = host_bits(lms[s % len(lms)])
            t1 = time.perf_counter()
            r = oracle.route(xb, wr, bias_np, k)
            oracle.expert_ffn(xb, inv.reshape(r["idx"].shape).astype(np.int32), r["w"],
                              sub["gate"], sub["up"], sub["down"])
            oracle.lmhead(hb, wl)
            samples.append(time.perf_counter() - t1)
            del wl, sub
        cpu_s = sum(samples) / n
        cpu_bytes = sum(layer_bytes[s % nl] for s in range(n)) / n + lm_bytes
        cores = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count()))
        cpu = {"value": round(cpu_bytes / cpu_s / 1e9, 3), "unit": "GB/s", "cores": cores,
               "kind": "oracle",
               "sample": f"{n} full steps (M={M} MoE layer route+experts+combine and "
                         f"lm_head argmax) in fp64, {cpu_s * 1e3:.0f} ms per step"}
        log(f"cpu oracle: {cpu_s * 1e3:.0f} ms/step on {cores} threads")

    res = {
        "metric": "cold-weight HBM GB/s (% of peak) + \u00b5s per MoE-layer verify step, M=6",
        "value": round(step_bytes_mean / (wall_ms * 1e-3) / 1e9, 1),
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
        "config": {"workload": f"moe_layer_verify_step_M{M}+lm_head_argmax",
                   "M": M, "hidden": H, "experts": E, "intermediate": I, "top_k": k,
                   "vocab": V, "layers_rotated": nl, "lm_head_copies": len(lms),
                   "zipf_alpha": args.zipf_alpha, "seeds": [synth.WEIGHT_SEED, synth.ACT_SEED]},
        "frac_of_hbm_peak": round(step_bytes_mean / (wall_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "gpu_ms_per_step_events": round(gpu_ms, 4),
        "moe_layer": {"us": round(layer_us_mean, 2), "GBps": round(layer_gbps, 1),
                      "frac": round(layer_gbps / HBM_PEAK_GBPS, 4),
                      "bytes": int(layer_bytes_mean), "distinct_experts_mean": sum(D) / len(D)},
        "lm_head": {"us": round(lm_us_mean, 2), "GBps": round(lm_gbps, 1),
                    "frac": round(lm_gbps / HBM_PEAK_GBPS, 4), "bytes": lm_bytes},
        "hbm_read_probe": {"GBps": round(probe_gbps, 1),
                           "frac": round(probe_gbps / HBM_PEAK_GBPS, 4),
                           "kernel": "moe_hbm_read_probe: grid-stride non-temporal 16-byte loads, "
                                     "256 x 256 threads, 8 in flight per thread",
                           "bytes_per_call": 2**30, "buffers_rotated": 4, "calls": 16},
        "router_gate_cold": {"us": round(route_us, 2),
                             "GBps": round(route_bytes / (route_us * 1e-6) / 1e9, 1),
                             "copies": R, "us_by_distinct_copies": gate_sweep},
        "moe_layer_other_widths": layer_sweep,
        "router_chain_rmsnorm": {"gate_us": round(route_norm_us, 2),
                                 "moe_layer_rmsnorm": layer_norm},
        "moe_layer_shared_expert": layer_shared,
        "fp8_weights": fp8,
        "roofline": {"kernel": "lmhead_kernel (lmhead_greedy_verify)", "bound": "hbm",
                     "achieved": round(lm_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(lm_gbps / HBM_PEAK_GBPS, 4), "traffic": traffic},
        "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
