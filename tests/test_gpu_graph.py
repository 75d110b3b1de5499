"""The verify step captured into a HIP graph through the raw C ABI and
replayed: every replay reproduces the eager calls' outputs bit for bit.

The step runs as captured graphs in the post ("The shape of a single-request
step", Fig. 3) and is timed in-graph ("Two fusions and a retune"). The
library enqueues kernels only (no host sync, no allocation, no memset), and
its workspace counters are back at zero after every call, so one captured
sequence can be replayed any number of times on the same workspaces. Each
replay here is preceded by eager work on the same workspaces and by a reset
of the outputs, and checked on its own."""
import ctypes

import numpy as np
import pytest
import torch

import moe_speculative_verify_amd as mv
import synth
from gpu_util import to_dev

pytestmark = pytest.mark.gpu


def say(*a):
    print("CASE", *a, flush=True)


def small_layer(H, E, I, layer):
    w = synth.layer_weights(H, E, I, layer=layer)
    return {key: to_dev(v) for key, v in w.items()}


class Step:
    """Inputs, outputs and raw argument tuples of one verify step: one MoE
    layer (moe_layer, or moe_layer_noalloc) and the lm_head verdict."""

    def __init__(self, L, M, H, I, E, k, V, layer, ws_layer, ws_lm, noalloc=False, zipf=None,
                 fp8=False):
        self.L, self.M, self.H, self.I, self.E, self.k, self.V = L, M, H, I, E, k, V
        self.w = small_layer(H, E, I, layer)
        self.fp8 = fp8
        if fp8:                                      # E4M3 codes, fp32 row scales
            for j, name in enumerate(("gate", "up", "down")):
                shape = (E, H, I) if name == "down" else (E, I, H)
                q, sc = synth.fp8_rows(shape, synth.WEIGHT_STD, 60 + layer, j + 1)
                self.w[name] = torch.from_numpy(q).cuda()
                self.w["s_" + name] = torch.from_numpy(sc).cuda()
            q, sc = synth.fp8_rows((V, H), synth.WEIGHT_STD, 65 + layer, 4)
            self.wlm8, self.slm8 = torch.from_numpy(q).cuda(), torch.from_numpy(sc).cuda()
        self.x = to_dev(synth.activations(M, H, seed=70 + layer))
        self.h = to_dev(synth.activations(M, H, seed=80 + layer))
        self.wlm = to_dev(synth.normal_bf16((V, H), synth.WEIGHT_STD, synth.WEIGHT_SEED, 90 + layer,
                                            synth.KIND["lm_head"]))
        self.bias = None if zipf is None else torch.from_numpy(synth.zipf_bias(E, zipf)).cuda()
        rng = np.random.default_rng(layer)
        self.chain = torch.from_numpy(rng.integers(0, V, size=M).astype(np.int32)).cuda()
        self.idx = torch.empty((M, k), dtype=torch.int32, device="cuda")
        self.tw = torch.empty((M, k), dtype=torch.float32, device="cuda")
        self.out = torch.empty((M, H), dtype=torch.float32, device="cuda")
        self.am = torch.empty(M, dtype=torch.int32, device="cuda")
        self.acc = torch.empty(2, dtype=torch.int32, device="cuda")
        self.ws_layer, self.ws_lm, self.noalloc = ws_layer, ws_lm, noalloc

    def outputs(self):
        return (self.idx, self.tw, self.out, self.am, self.acc)

    def poison(self):
        for t in self.outputs():
            t.view(torch.int32).fill_(-7)

    def enqueue(self, stream):
        L, M, H, I, E, k = self.L, self.M, self.H, self.I, self.E, self.k
        b = None if self.bias is None else self.bias.data_ptr()
        if self.fp8:
            w = self.w
            rc = L.moe_layer_fp8(self.x.data_ptr(), w["router"].data_ptr(), b,
                                 w["gate"].data_ptr(), w["s_gate"].data_ptr(), w["up"].data_ptr(),
                                 w["s_up"].data_ptr(), w["down"].data_ptr(),
                                 w["s_down"].data_ptr(), M, H, I, E, k, self.idx.data_ptr(),
                                 self.tw.data_ptr(), self.out.data_ptr(), self.ws_layer.data_ptr(),
                                 ctypes.c_size_t(self.ws_layer.numel()), stream)
            assert rc == 0, mv.status_str(rc)
            rc = L.lmhead_greedy_verify_fp8(self.h.data_ptr(), self.wlm8.data_ptr(),
                                            self.slm8.data_ptr(), self.chain.data_ptr(), M, H,
                                            self.V, self.am.data_ptr(), None, self.acc.data_ptr(),
                                            self.ws_lm.data_ptr(),
                                            ctypes.c_size_t(self.ws_lm.numel()), stream)
            assert rc == 0, mv.status_str(rc)
            return
        a = [self.x.data_ptr(), self.w["router"].data_ptr(), b, self.w["gate"].data_ptr(),
             self.w["up"].data_ptr(), self.w["down"].data_ptr(), M, H, I, E, k,
             self.idx.data_ptr(), self.tw.data_ptr(), self.out.data_ptr()]
        if self.noalloc:
            rc = L.moe_layer_noalloc(*a, stream)
        else:
            rc = L.moe_layer(*a, self.ws_layer.data_ptr(), ctypes.c_size_t(self.ws_layer.numel()),
                             stream)
        assert rc == 0, mv.status_str(rc)
        rc = L.lmhead_greedy_verify(self.h.data_ptr(), self.wlm.data_ptr(), self.chain.data_ptr(),
                                    M, H, self.V, self.am.data_ptr(), None, self.acc.data_ptr(),
                                    self.ws_lm.data_ptr(), ctypes.c_size_t(self.ws_lm.numel()),
                                    stream)
        assert rc == 0, mv.status_str(rc)


def run_graph_case(M, H, I, E, k, V, nsteps, noalloc_step=None, zipf=None, fp8=False):
    L = mv.lib()
    ws_layer = torch.zeros(L.moe_layer_workspace_bytes(M, H, I, E, k), dtype=torch.uint8,
                           device="cuda")
    ws_lm = torch.zeros(L.lmhead_argmax_workspace_bytes(M, V), dtype=torch.uint8, device="cuda")
    steps = [Step(L, M, H, I, E, k, V, layer=s, ws_layer=ws_layer, ws_lm=ws_lm,
                  noalloc=(s == noalloc_step), zipf=zipf, fp8=fp8) for s in range(nsteps)]
    cur = torch.cuda.current_stream().cuda_stream
    # eager reference (also the warm-up: attributes and the static scratch
    # address are set up outside the capture)
    for st in steps:
        st.poison()
        st.enqueue(cur)
    torch.cuda.synchronize()
    ref = [[t.clone() for t in st.outputs()] for st in steps]

    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    with torch.cuda.graph(g, stream=cap):
        for st in steps:
            st.enqueue(cap.cuda_stream)
    torch.cuda.synchronize()
    for rep in range(4):
        say(f"graph M={M} H={H} I={I} E={E} k={k} V={V} steps={nsteps} replay {rep}")
        # eager work on the same workspaces between replays: the step in
        # reverse order, whose outputs must match too
        for st in reversed(steps):
            st.poison()
            st.enqueue(cur)
        torch.cuda.synchronize()
        for st, r in zip(steps, ref):
            for a, b in zip(st.outputs(), r):
                assert torch.equal(a, b), "eager rerun"
            st.poison()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for s, (st, r) in enumerate(zip(steps, ref)):
            for name, a, b in zip(("topk_idx", "topk_w", "out", "argmax", "accept"),
                                  st.outputs(), r):
                assert torch.equal(a, b), f"replay {rep} step {s}: {name} differs from eager"
    # the header counters are back at zero after the replays
    assert int(ws_layer[:4096].count_nonzero()) == 0
    assert int(ws_lm[:4096].count_nonzero()) == 0


def test_graph_replay_equals_eager_gemv_regime():
    # M = 6 verify width, GEMV down kernel; one step uses moe_layer_noalloc
    run_graph_case(6, 512, 256, 64, 8, 3001, nsteps=3, noalloc_step=1)


def test_graph_replay_equals_eager_mfma_regime():
    # M = 16 block verify with Zipf-skewed routing: M*k*I*2 bytes of
    # activations above the GEMV down kernel's LDS, the MFMA down kernel runs
    run_graph_case(16, 512, 1024, 32, 8, 2048, nsteps=2, zipf=1.0)


def test_graph_replay_equals_eager_one_token():
    run_graph_case(1, 256, 128, 16, 2, 1000, nsteps=3, noalloc_step=2)


def test_graph_replay_equals_eager_fp8_shared_experts():
    # fp8 layer and fp8 lm_head verdict at M = 16 with Zipf-skewed routing:
    # experts that four or more pairs share run both projections on the
    # matrix cores inside the captured graph
    run_graph_case(16, 512, 256, 24, 8, 2048, nsteps=2, zipf=1.0, fp8=True)
