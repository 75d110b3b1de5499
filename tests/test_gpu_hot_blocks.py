"""GPU parity of experts that several verify tokens share. With fp8
weights a column block of at least 4 pairs runs the up projection on the
matrix cores (8-row units: 8 gate and 8 up rows against the block's pairs)
instead of one-row GEMV units, and the down projection's blocks of it on the
matrix cores too (a workgroup's rows against the block's pairs); with bf16
weights every block stays on the GEMV paths, each pair paying its own dot
products. The routing is planted so
that the number of pairs per expert is known: blocks of exactly 4 (the
threshold) and 3 (below it), 16 (a full block), an odd number of hot blocks
(the last one stays on the GEMV path), ragged K tails, I not a multiple of
64, the shared expert's block, and more than 64 pairs (the histogram
grouping). Outputs against the fp64 oracle within 1e-2 * max|ref| per
tensor.
"""
import numpy as np
import pytest
import torch

import moe_speculative_verify_amd as mv
import oracle
import synth
from gpu_util import assert_close, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    mv.lib()
    yield
    torch.cuda.synchronize()


def say(*a):
    print("CASE", *a, flush=True)


def planted_routing(M, E, k, counts, seed):
    """Token t's k distinct experts: expert e (e < len(counts)) is given to
    the counts[e] tokens with the fewest experts so far, so it serves exactly
    counts[e] pairs; every other slot gets an expert of its own, from E - 1
    down. Returns (idx [M,k] int32, weights [M,k] float32 summing to one)."""
    g = np.random.default_rng(seed)
    assert sum(counts) <= M * k
    assert M * k - sum(counts) <= E - len(counts), "not enough single-use experts"
    idx = np.full((M, k), -1, np.int32)
    fill = np.zeros(M, np.int64)
    for e, c in enumerate(counts):
        for t in np.argsort(fill, kind="stable")[:c]:
            assert fill[t] < k
            idx[t, fill[t]] = e
            fill[t] += 1
    spare = list(range(E - 1, len(counts) - 1, -1))
    for t in range(M):
        while fill[t] < k:
            idx[t, fill[t]] = spare.pop(0)
            fill[t] += 1
        g.shuffle(idx[t])
    for e, c in enumerate(counts):
        assert int((idx == e).sum()) == c
    w = g.uniform(0.1, 1.0, (M, k)).astype(np.float32)
    w /= w.sum(axis=1, keepdims=True)
    return idx, w


HOT_CASES = [
    # M, H, I, E, k, pairs per planted expert
    (16, 520, 40, 48, 3, (16, 9, 4, 3)),       # blocks of 16, 9, 4 and 3 pairs; K tail of one chunk
    (8, 256, 64, 40, 4, (8, 8, 4, 4, 3)),      # two blocks exactly at the fp8 threshold
    (16, 2560, 128, 64, 6, (16, 16, 12, 5)),   # the model's width; 96 pairs (histogram)
    (6, 1032, 1032, 24, 2, (6, 6)),            # every token on both experts; K tail
]


@pytest.mark.parametrize("M,H,I,E,k,counts", HOT_CASES)
def test_shared_blocks_bf16(M, H, I, E, k, counts):
    say("shared blocks bf16", M, H, I, E, k, counts)
    x = synth.activations(M, H, seed=7000 + H)
    w = synth.layer_weights(H, E, I, seed=synth.WEIGHT_SEED + 70 + I)
    idx, tw = planted_routing(M, E, k, counts, 7100 + M)
    out = mv.moe_expert_ffn(to_dev(x), torch.from_numpy(idx).cuda(), torch.from_numpy(tw).cuda(),
                            to_dev(w["gate"]), to_dev(w["up"]), to_dev(w["down"]))
    torch.cuda.synchronize()
    ref = oracle.expert_ffn(x, idx, tw.astype(np.float64), w["gate"], w["up"], w["down"])
    assert_close(out.cpu().numpy(), ref, "out")


def _fp8_host(H, I, E, seed):
    qg, sg = synth.fp8_rows((E, I, H), synth.WEIGHT_STD, seed, 1)
    qu, su = synth.fp8_rows((E, I, H), synth.WEIGHT_STD, seed, 2)
    qd, sd = synth.fp8_rows((E, H, I), synth.WEIGHT_STD, seed, 3)
    return dict(gate=qg, s_gate=sg, up=qu, s_up=su, down=qd, s_down=sd)


FP8_HOT_CASES = [
    # M, H, I, E, k, pairs per planted expert
    (16, 528, 48, 48, 3, (16, 9, 4, 3)),       # up: 2 hot blocks on the MFMA, one stays GEMV (down: all 3); 8 rows in the last down workgroup
    (12, 2560, 64, 40, 4, (12, 12, 7, 4)),     # the model's width: 3 K blocks of codes, the last partial
    (16, 1040, 1040, 24, 2, (16, 5, 5)),       # 1040 columns: a 16-code tail chunk in both projections; odd hot count
    (8, 256, 64, 40, 4, (8, 8, 4, 4, 3)),      # 4 hot blocks, two exactly at the threshold
    (16, 2560, 128, 64, 6, (16, 16, 12, 5)),   # 96 pairs (histogram grouping), 4 hot blocks
]


@pytest.mark.parametrize("M,H,I,E,k,counts", FP8_HOT_CASES)
def test_hot_blocks_fp8(M, H, I, E, k, counts):
    say("hot blocks fp8", M, H, I, E, k, counts)
    x = synth.activations(M, H, seed=7200 + H)
    w = _fp8_host(H, I, E, 7300 + I)
    idx, tw = planted_routing(M, E, k, counts, 7400 + M)

    def dev(a):
        a = np.ascontiguousarray(a)
        return torch.from_numpy(a).cuda()
    out = mv.moe_expert_ffn_fp8(to_dev(x), dev(idx), dev(tw), dev(w["gate"]), dev(w["s_gate"]),
                                dev(w["up"]), dev(w["s_up"]), dev(w["down"]), dev(w["s_down"]))
    torch.cuda.synchronize()
    ref = oracle.expert_ffn_fp8(x, idx, tw, w["gate"], w["s_gate"], w["up"], w["s_up"],
                                w["down"], w["s_down"])
    assert_close(out.cpu().numpy(), ref, "out")


def test_shared_expert_with_shared_block():
    """The shared expert's block holds every token (6 pairs at M = 6) beside a
    routed expert that every token uses too (bf16: the GEMV path)."""
    M, H, I, E, k = 6, 264, 72, 20, 3
    say("hot blocks shared", M, H, I, E, k)
    x = synth.activations(M, H, seed=7500)
    w = synth.layer_weights(H, E, I, seed=synth.WEIGHT_SEED + 75)
    sw = dict(gate=synth.normal_bf16((I, H), synth.WEIGHT_STD, 7501, 71),
              up=synth.normal_bf16((I, H), synth.WEIGHT_STD, 7501, 72),
              down=synth.normal_bf16((H, I), synth.WEIGHT_STD, 7501, 73))
    idx, tw = planted_routing(M, E, k, (6, 2), 7502)
    out = mv.moe_expert_ffn_shared(to_dev(x), torch.from_numpy(idx).cuda(),
                                   torch.from_numpy(tw).cuda(), to_dev(w["gate"]),
                                   to_dev(w["up"]), to_dev(w["down"]), to_dev(sw["gate"]),
                                   to_dev(sw["up"]), to_dev(sw["down"]))
    torch.cuda.synchronize()
    idx2 = np.concatenate([idx, np.full((M, 1), E, np.int32)], axis=1)
    w2 = np.concatenate([tw.astype(np.float64), np.ones((M, 1))], axis=1)
    ref = oracle.expert_ffn(x, idx2, w2, np.concatenate([w["gate"], sw["gate"][None]]),
                            np.concatenate([w["up"], sw["up"][None]]),
                            np.concatenate([w["down"], sw["down"][None]]))
    assert_close(out.cpu().numpy(), ref, "out")


def test_hot_token_alone_within_tolerance():
    """fp8: a token whose experts are hot in a 16-token call (matrix cores)
    and the same token alone (GEMV) agree within the parity tolerance, the
    two paths summing in different orders; 16 identical tokens give 16
    bitwise-equal rows."""
    M, H, I, E, k = 16, 512, 64, 32, 4
    say("hot blocks: token alone", M, H, I, E, k)
    x = synth.activations(M, H, seed=7600)
    w = _fp8_host(H, I, E, 7602)
    idx, tw = planted_routing(M, E, k, (16, 16, 8), 7601)

    def dev(a):
        return torch.from_numpy(np.ascontiguousarray(a)).cuda()
    dw = [dev(w[n]) for n in ("gate", "s_gate", "up", "s_up", "down", "s_down")]

    def ffn(xx, ii, ww):
        return mv.moe_expert_ffn_fp8(to_dev(xx), dev(ii), dev(ww), *dw).cpu().numpy()
    full = ffn(x, idx, tw)
    for t in (0, 9, 15):
        one = ffn(x[t:t + 1], idx[t:t + 1], tw[t:t + 1])
        assert_close(full[t], one[0], f"token {t} in the call against alone")
    same = ffn(np.repeat(x[:1], M, axis=0), np.repeat(idx[:1], M, axis=0),
               np.repeat(tw[:1], M, axis=0))
    for t in range(M):
        assert np.array_equal(same[t], same[0])
    assert_close(same[0], ffn(x[:1], idx[:1], tw[:1])[0], "identical tokens against alone")
