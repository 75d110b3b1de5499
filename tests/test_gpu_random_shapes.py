"""Seeded random shapes through the C ABI against the fp64 CPU oracle.

Each case draws its own sizes inside the header's limits (small enough for
the oracle to finish in a second or two), so that the kernels' ragged edges
meet in combinations no hand-picked case covers: unit counts that end
anywhere in the up kernel's dealing periods, column blocks of one to sixteen
pairs in every grouping path (with and without the shared expert, whose
blocks go first), K tails of every length, both down kernels, and lm_head
tile counts and K blocks that leave partial tiles and partial rings, and
whole layers whose selection runs in the up kernel (ragged E, one to four
slices of H; bf16, and fp8 with experts that four or more pairs share on
the matrix cores). The draws come from one fixed seed; the case list is the same
on every run.

Acceptance as in every parity test: expert-FFN outputs within
1e-2 * max|ref|; argmax exact except at oracle-flagged near-ties, where the
GPU's choice must be a valid argmax within the band; the verdict exact
given the GPU's own argmax.
"""
import numpy as np
import pytest
import torch

import moe_speculative_verify_amd as mv
import oracle
import synth
from gpu_util import TIE_BAND, assert_close, check_tie_rows, compare_route, to_dev

pytestmark = pytest.mark.gpu

SEED = 20261202


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    mv.lib()
    yield
    torch.cuda.synchronize()


def say(*a):
    print("CASE", *a, flush=True)


def _mult(rng, lo, hi, m):
    return int(rng.integers(lo // m, hi // m + 1)) * m


def _ffn_cases(n):
    rng = np.random.default_rng(SEED)
    cases = []
    for c in range(n):
        kind = ("bf16", "fp8", "shared")[c % 3]
        m = 16 if kind == "fp8" else 8
        M = int(rng.integers(1, 17))
        E = int(rng.integers(2, 97))
        k = int(rng.integers(1, min(E, 16) + 1))
        while M * (k + (kind == "shared")) > 256:
            k -= 1
        H = _mult(rng, m, 1024, m)
        I = _mult(rng, m, 3000, m)
        while H * I > 1_200_000:                     # keep the oracle quick
            I = max(m, (I // 2) // m * m)
        skew = float(rng.choice([0.0, 1.0]))
        cases.append((c, kind, M, H, I, E, k, skew))
    return cases


def _u8(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.uint8)).cuda()


def _f32(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda()


@pytest.mark.parametrize("c,kind,M,H,I,E,k,skew", _ffn_cases(30))
def test_random_expert_ffn(c, kind, M, H, I, E, k, skew):
    say("random expert_ffn", c, kind, M, H, I, E, k, skew)
    x = synth.activations(M, H, seed=7000 + c)
    idx, tw = synth.random_routing(M, E, k, 7100 + c, skew)
    idx_d, tw_d = torch.from_numpy(idx).cuda(), torch.from_numpy(tw).cuda()
    if kind == "fp8":
        qg, sg = synth.fp8_rows((E, I, H), synth.WEIGHT_STD, 7200 + c, 1)
        qu, su = synth.fp8_rows((E, I, H), synth.WEIGHT_STD, 7200 + c, 2)
        qd, sd = synth.fp8_rows((E, H, I), synth.WEIGHT_STD, 7200 + c, 3)
        out = mv.moe_expert_ffn_fp8(to_dev(x), idx_d, tw_d, _u8(qg), _f32(sg), _u8(qu),
                                    _f32(su), _u8(qd), _f32(sd))
        torch.cuda.synchronize()
        ref = oracle.expert_ffn_fp8(x, idx, tw, qg, sg, qu, su, qd, sd)
    else:
        w = synth.layer_weights(H, E, I, seed=synth.WEIGHT_SEED + 7300 + c)
        args = (to_dev(x), idx_d, tw_d, to_dev(w["gate"]), to_dev(w["up"]), to_dev(w["down"]))
        if kind == "shared":
            sg = synth.normal_bf16((I, H), synth.WEIGHT_STD, 7400 + c, 1)
            su = synth.normal_bf16((I, H), synth.WEIGHT_STD, 7400 + c, 2)
            sd = synth.normal_bf16((H, I), synth.WEIGHT_STD, 7400 + c, 3)
            out = mv.moe_expert_ffn_shared(*args, to_dev(sg), to_dev(su), to_dev(sd))
            torch.cuda.synchronize()
            # the shared expert is slot k of every token, expert id E, weight 1
            idx2 = np.concatenate([idx, np.full((M, 1), E, np.int32)], axis=1)
            tw2 = np.concatenate([np.asarray(tw, np.float64), np.ones((M, 1))], axis=1)
            ref = oracle.expert_ffn(x, idx2, tw2, np.concatenate([w["gate"], sg[None]]),
                                    np.concatenate([w["up"], su[None]]),
                                    np.concatenate([w["down"], sd[None]]))
        else:
            out = mv.moe_expert_ffn(*args)
            torch.cuda.synchronize()
            ref = oracle.expert_ffn(x, idx, tw, w["gate"], w["up"], w["down"])
    assert_close(out.cpu().numpy(), ref, "out")


def _lm_cases(n):
    rng = np.random.default_rng(SEED + 1)
    cases = []
    for c in range(n):
        w8 = bool(c % 2)
        M = int(rng.integers(1, 17))
        H = _mult(rng, 16 if w8 else 8, 1536, 16 if w8 else 8)
        V = int(rng.integers(1, 9000))
        cases.append((c, w8, M, H, V))
    return cases


@pytest.mark.parametrize("c,w8,M,H,V", _lm_cases(16))
def test_random_lmhead_verdict(c, w8, M, H, V):
    say("random lm_head + verdict", c, w8, M, H, V)
    h = synth.activations(M, H, seed=7500 + c)
    rng = np.random.default_rng(SEED + 100 + c)
    if w8:
        q, s = synth.fp8_rows((V, H), synth.WEIGHT_STD, 7600 + c, 1)
        ref = oracle.lmhead_fp8(h, q, s)
    else:
        wl = synth.normal_bf16((V, H), synth.WEIGHT_STD, 7600 + c, 1)
        ref = oracle.lmhead(h, wl)
    # a chain that agrees with the oracle's argmax for a random prefix
    n_ok = int(rng.integers(0, M))
    tokens = np.zeros(M, np.int32)
    tokens[0] = int(rng.integers(0, V))
    for i in range(1, M):
        tokens[i] = ref["tok"][i - 1] if i <= n_ok else int(rng.integers(0, V))
    tok_d = torch.from_numpy(tokens).cuda()
    if w8:
        am, acc, ml = mv.lmhead_greedy_verify_fp8(to_dev(h), _u8(q), _f32(s), tok_d, want_max=True)
    else:
        am, acc, ml = mv.lmhead_greedy_verify(to_dev(h), to_dev(wl), tok_d, want_max=True)
    torch.cuda.synchronize()
    am, acc, ml = am.cpu().numpy(), acc.cpu().numpy(), ml.cpu().numpy()
    for t in range(M):
        if am[t] != ref["tok"][t]:
            assert ref["gap"][t] < TIE_BAND, f"token {t}: {am[t]} != {ref['tok'][t]}"
            assert 0 <= am[t] < V
    assert_close(ml, ref["zmax"], "max_logit")
    n, bonus = oracle.greedy_verdict(tokens, am)
    assert (acc[0], acc[1]) == (n, bonus)


def _layer_cases(n):
    rng = np.random.default_rng(SEED + 2)
    cases = []
    for c in range(n):
        M = int(rng.integers(1, 17))
        E = int(rng.integers(2, 513))                # E <= 512: the up kernel selects
        k = int(rng.integers(1, min(E, 16) + 1))
        H = _mult(rng, 8, 1024, 8)
        I = _mult(rng, 8, 1024, 8)
        while E * H * I > 40_000_000:               # keep the host weights small
            E = max(k, E // 2)
        alpha = [None, 0.5, 1.0][c % 3]
        cases.append((c, M, H, I, E, k, alpha))
    return cases


@pytest.mark.parametrize("c,M,H,I,E,k,alpha", _layer_cases(12))
def test_random_layer(c, M, H, I, E, k, alpha):
    """moe_layer (selection inside the up kernel from the router kernel's
    partial logits) against the oracle's route and FFN: ids and weights
    exact away from near-ties, outputs within tolerance; a near-tie row's
    output checked against the oracle FFN on the GPU's own selection."""
    say("random layer", c, M, H, I, E, k, alpha)
    x = synth.activations(M, H, seed=7700 + c)
    w = synth.layer_weights(H, E, I, seed=synth.WEIGHT_SEED + 7800 + c)
    bias = None if alpha is None else synth.zipf_bias(E, alpha)
    b = None if bias is None else torch.from_numpy(bias).cuda()
    gi, gw, go = mv.moe_layer(to_dev(x), to_dev(w["router"]), to_dev(w["gate"]), to_dev(w["up"]),
                              to_dev(w["down"]), k, b)
    torch.cuda.synchronize()
    gi, gw, go = gi.cpu().numpy(), gw.cpu().numpy(), go.cpu().numpy()
    ref = oracle.route(x, w["router"], bias, k)
    same = compare_route(gi, gw, None, ref, k)
    out = oracle.expert_ffn(x, ref["idx"], ref["w"], w["gate"], w["up"], w["down"])
    assert_close(go[same], out[same], "out")
    check_tie_rows(x, gi, gw, go, ref, lambda xr, ids, tw: oracle.expert_ffn(
        xr, ids, tw, w["gate"], w["up"], w["down"]))


def _layer8_cases(n):
    rng = np.random.default_rng(SEED + 3)
    cases = []
    for c in range(n):
        M = int(rng.integers(4, 17))                 # four or more pairs can share a block
        E = int(rng.integers(2, 129))
        k = int(rng.integers(1, min(E, 16) + 1))
        H = _mult(rng, 16, 1024, 16)
        I = _mult(rng, 16, 1024, 16)
        while E * H * I > 40_000_000:
            E = max(k, E // 2)
        alpha = [1.0, 0.5, None][c % 3]
        cases.append((c, M, H, I, E, k, alpha))
    return cases


@pytest.mark.parametrize("c,M,H,I,E,k,alpha", _layer8_cases(9))
def test_random_layer_fp8(c, M, H, I, E, k, alpha):
    """moe_layer_fp8: the selection inside the fp8 up kernel, then both
    projections with the experts that four or more of the call's pairs share
    on the matrix cores and the rest on the GEMV paths (the skewed draws
    make such experts common), against the oracle's route and fp8 FFN."""
    say("random layer fp8", c, M, H, I, E, k, alpha)
    x = synth.activations(M, H, seed=7900 + c)
    router = synth.normal_bf16((E, H), synth.WEIGHT_STD, synth.WEIGHT_SEED + 7950 + c, 0)
    w = {}
    for j, name in enumerate(("gate", "up", "down")):
        shape = (E, H, I) if name == "down" else (E, I, H)
        w[name], w["s_" + name] = synth.fp8_rows(shape, synth.WEIGHT_STD, 8000 + c, j + 1)
    bias = None if alpha is None else synth.zipf_bias(E, alpha)
    b = None if bias is None else torch.from_numpy(bias).cuda()
    gi, gw, go = mv.moe_layer_fp8(to_dev(x), to_dev(router), _u8(w["gate"]), _f32(w["s_gate"]),
                                  _u8(w["up"]), _f32(w["s_up"]), _u8(w["down"]),
                                  _f32(w["s_down"]), k, b)
    torch.cuda.synchronize()
    gi, gw, go = gi.cpu().numpy(), gw.cpu().numpy(), go.cpu().numpy()
    ref = oracle.route(x, router, bias, k)
    same = compare_route(gi, gw, None, ref, k)

    def ffn8(xr, ids, tw):
        return oracle.expert_ffn_fp8(xr, ids, tw, w["gate"], w["s_gate"], w["up"], w["s_up"],
                                     w["down"], w["s_down"])
    assert_close(go[same], ffn8(x, ref["idx"], ref["w"])[same], "out")
    check_tie_rows(x, gi, gw, go, ref, ffn8)
