"""Bounds and workspace hygiene on the GPU.

Canary words sit past the end of every output and past the queried size of
every workspace at ragged shapes: no call may write beyond what it owns.
One workspace reused by calls of shrinking shapes must give the results of
fresh ones (whatever a larger call left past the header -- its activations,
partial logits or keys -- must never be read as a counter or as data by a
smaller one), with the header's counters back at zero after every call. The workspace
clear zeroes exactly its bytes, also replayed from a graph.
"""
import numpy as np
import pytest
import torch

import moe_speculative_verify_amd as mv
import synth
from gpu_util import device_layer, to_dev

pytestmark = pytest.mark.gpu

HEADER = 4096
CANARY_I32 = 0x5A5AA5A5
CANARY_U8 = 0xC3


def say(*a):
    print("CASE", *a, flush=True)


def padded(shape, dtype, extra=64):
    """A tensor view of `shape` whose storage continues with `extra` canary
    elements."""
    n = int(np.prod(shape))
    base = torch.empty(n + extra, dtype=dtype, device="cuda")
    base.view(torch.int32 if dtype in (torch.int32, torch.float32) else torch.int16).fill_(
        CANARY_I32 if dtype in (torch.int32, torch.float32) else 0x5A5A)
    return base[:n].view(shape), base


def canary_intact(base, n):
    tail = base[n:]
    if tail.dtype in (torch.int32, torch.float32):
        return bool((tail.view(torch.int32) == CANARY_I32).all())
    return bool((tail.view(torch.int16) == 0x5A5A).all())


def workspace(nbytes, extra=4096):
    ws = torch.zeros(nbytes + extra, dtype=torch.uint8, device="cuda")
    ws[nbytes:] = CANARY_U8
    return ws


def ws_ok(ws, nbytes):
    return bool((ws[nbytes:] == CANARY_U8).all()) and int(ws[:HEADER].count_nonzero()) == 0


@pytest.mark.parametrize("M,H,I,E,k", [(3, 264, 136, 20, 4), (1, 1032, 256, 12, 3),
                                       (9, 520, 72, 100, 6), (16, 256, 1024, 16, 8)])
def test_layer_and_ffn_stay_in_bounds(M, H, I, E, k):
    say("canaries layer/ffn", M, H, I, E, k)
    w = synth.layer_weights(H, E, I, seed=synth.WEIGHT_SEED + 31 * M + H)
    dw = {key: to_dev(v) for key, v in w.items()}
    x = to_dev(synth.activations(M, H, seed=3000 + M))
    idx, ib = padded((M, k), torch.int32)
    tw, wb = padded((M, k), torch.float32)
    out, ob = padded((M, H), torch.float32)
    nb = mv.moe_layer_workspace_bytes(M, H, I, E, k)
    ws = workspace(nb)
    mv.moe_layer(x, dw["router"], dw["gate"], dw["up"], dw["down"], k, out=(idx, tw, out),
                 workspace=ws[:nb])
    torch.cuda.synchronize()
    assert canary_intact(ib, M * k) and canary_intact(wb, M * k) and canary_intact(ob, M * H)
    assert ws_ok(ws, nb)
    # the FFN alone on the layer's ids, with its own workspace size
    out2, ob2 = padded((M, H), torch.float32)
    nf = mv.moe_expert_ffn_workspace_bytes(M, H, I, E, k)
    wf = workspace(nf)
    mv.moe_expert_ffn(x, idx, tw, dw["gate"], dw["up"], dw["down"], out=out2, workspace=wf[:nf])
    torch.cuda.synchronize()
    assert canary_intact(ob2, M * H) and ws_ok(wf, nf)
    assert torch.equal(out, out2)



@pytest.mark.parametrize("M,H,I,E,k", [(16, 528, 48, 10, 5), (5, 272, 1040, 6, 4),
                                       (1, 1040, 256, 12, 3), (12, 256, 2064, 40, 8)])
def test_layer_fp8_stays_in_bounds(M, H, I, E, k):
    """moe_layer_fp8 then the fp8 lm_head verdict at ragged shapes, with few
    experts for many pairs (the matrix-core units of shared experts, with
    K tails and a ragged last down workgroup), canaries after every output
    and workspace."""
    say("canaries layer fp8", M, H, I, E, k)
    router = to_dev(synth.normal_bf16((E, H), synth.WEIGHT_STD, 3500 + H, 0))
    d = {}
    for j, name in enumerate(("gate", "up", "down")):
        shape = (E, H, I) if name == "down" else (E, I, H)
        q, sc = synth.fp8_rows(shape, synth.WEIGHT_STD, 3501 + I, j + 1)
        d[name], d["s_" + name] = torch.from_numpy(q).cuda(), torch.from_numpy(sc).cuda()
    x = to_dev(synth.activations(M, H, seed=3502 + M))
    idx, ib = padded((M, k), torch.int32)
    tw, wb = padded((M, k), torch.float32)
    out, ob = padded((M, H), torch.float32)
    nb = mv.moe_layer_workspace_bytes(M, H, I, E, k)
    ws = workspace(nb)
    mv.moe_layer_fp8(x, router, d["gate"], d["s_gate"], d["up"], d["s_up"], d["down"],
                     d["s_down"], k, out=(idx, tw, out), workspace=ws[:nb])
    torch.cuda.synchronize()
    assert canary_intact(ib, M * k) and canary_intact(wb, M * k) and canary_intact(ob, M * H)
    assert ws_ok(ws, nb)
    V = 3 * 16 + 5                                    # a partial last tile
    q, sc = synth.fp8_rows((V, H), synth.WEIGHT_STD, 3503, V)
    am, ab = padded((M,), torch.int32)
    ml, mb = padded((M,), torch.float32)
    acc, cb = padded((2,), torch.int32)
    nl = mv.lmhead_argmax_workspace_bytes(M, V)
    wl = workspace(nl)
    chain = torch.zeros(M, dtype=torch.int32, device="cuda")
    mv.lmhead_greedy_verify_fp8(to_dev(synth.activations(M, H, seed=3504)),
                                torch.from_numpy(q).cuda(), torch.from_numpy(sc).cuda(), chain,
                                want_max=True, out=(am, acc, ml), workspace=wl[:nl])
    torch.cuda.synchronize()
    assert canary_intact(ab, M) and canary_intact(mb, M) and canary_intact(cb, 2)
    assert ws_ok(wl, nl)

@pytest.mark.parametrize("M,H,V", [(3, 264, 777), (16, 256, 4099), (1, 2560, 65)])
def test_lmhead_stays_in_bounds(M, H, V):
    say("canaries lm_head", M, H, V)
    h = to_dev(synth.activations(M, H, seed=3100 + V))
    wl = to_dev(synth.normal_bf16((V, H), synth.WEIGHT_STD, 3101, V))
    am, ab = padded((M,), torch.int32)
    ml, mb = padded((M,), torch.float32)
    acc, cb = padded((2,), torch.int32)
    nb = mv.lmhead_argmax_workspace_bytes(M, V)
    ws = workspace(nb)
    chain = torch.zeros(M, dtype=torch.int32, device="cuda")
    mv.lmhead_greedy_verify(h, wl, chain, want_max=True, out=(am, acc, ml), workspace=ws[:nb])
    torch.cuda.synchronize()
    assert canary_intact(ab, M) and canary_intact(mb, M) and canary_intact(cb, 2)
    assert ws_ok(ws, nb)


def test_ffn_workspace_reused_by_shrinking_shapes():
    """moe_expert_ffn (bf16 and fp8) and moe_layer on one workspace at
    shrinking shapes: each result equals the same call on a fresh zero-filled
    workspace and the header is zero after every call."""
    say("ffn workspace reused by shrinking shapes")
    shapes = [(9, 512, 1024, 64, 8), (2, 16, 16, 3, 2), (6, 272, 144, 20, 4), (1, 256, 128, 16, 2)]
    big = max(mv.moe_layer_workspace_bytes(M, H, I, E, k) for M, H, I, E, k in shapes)
    shared = torch.zeros(big, dtype=torch.uint8, device="cuda")
    for M, H, I, E, k in shapes:
        say("  shape", M, H, I, E, k)
        w = synth.layer_weights(H, E, I, seed=synth.WEIGHT_SEED + 11 * H + E)
        dw = {key: to_dev(v) for key, v in w.items()}
        x = to_dev(synth.activations(M, H, seed=3200 + M))
        idx_np, tw_np = synth.random_routing(M, E, k, 3300 + M)
        idx, tw = torch.from_numpy(idx_np).cuda(), torch.from_numpy(tw_np).cuda()
        a = mv.moe_expert_ffn(x, idx, tw, dw["gate"], dw["up"], dw["down"],
                              workspace=torch.zeros(big, dtype=torch.uint8, device="cuda"))
        b = mv.moe_expert_ffn(x, idx, tw, dw["gate"], dw["up"], dw["down"], workspace=shared)
        torch.cuda.synchronize()
        assert torch.equal(a, b) and int(shared[:HEADER].count_nonzero()) == 0
        la = mv.moe_layer(x, dw["router"], dw["gate"], dw["up"], dw["down"], k,
                          workspace=torch.zeros(big, dtype=torch.uint8, device="cuda"))
        lb = mv.moe_layer(x, dw["router"], dw["gate"], dw["up"], dw["down"], k, workspace=shared)
        torch.cuda.synchronize()
        for ta, tb in zip(la, lb):
            assert torch.equal(ta, tb)
        assert int(shared[:HEADER].count_nonzero()) == 0
        if H % 16 == 0 and I % 16 == 0:
            q = {key: synth.fp8_rows(w[key].shape, synth.WEIGHT_STD, 3400 + H, i)
                 for i, key in enumerate(("gate", "up", "down"))}
            d8 = [torch.from_numpy(np.ascontiguousarray(v)).cuda() for key in ("gate", "up", "down")
                  for v in q[key]]
            a8 = mv.moe_expert_ffn_fp8(x, idx, tw, *d8,
                                       workspace=torch.zeros(big, dtype=torch.uint8, device="cuda"))
            b8 = mv.moe_expert_ffn_fp8(x, idx, tw, *d8, workspace=shared)
            torch.cuda.synchronize()
            assert torch.equal(a8, b8) and int(shared[:HEADER].count_nonzero()) == 0


@pytest.mark.parametrize("nbytes", [16, 4096, 4096 + 48, 3 * 1024 * 1024 + 16])
def test_workspace_clear_fills_exactly_its_bytes(nbytes):
    """moe_workspace_clear zeroes exactly `bytes` (ragged against its fill
    kernel's 16-byte stores and grid), eagerly and as a captured graph
    replayed several times, each replay after an eager re-poisoning."""
    say("workspace clear", nbytes)
    ws = workspace(nbytes)
    ws[:nbytes] = 0xA7
    mv.moe_workspace_clear(ws[:nbytes])
    torch.cuda.synchronize()
    assert int(ws[:nbytes].count_nonzero()) == 0
    assert bool((ws[nbytes:] == CANARY_U8).all())
    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    with torch.cuda.graph(g, stream=cap):
        mv.moe_workspace_clear(ws[:nbytes], stream=cap)
    for rep in range(3):
        ws[:nbytes] = 0x5C + rep
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert int(ws[:nbytes].count_nonzero()) == 0, f"replay {rep}"
        assert bool((ws[nbytes:] == CANARY_U8).all()), f"replay {rep}"
