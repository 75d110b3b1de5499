"""GPU parity: the HIP path through the C ABI against the fp64 CPU oracle.

Every case prints its name and shape before it touches the GPU. Indices must
be bit-exact except where the oracle flags a near-tie (fp64 gap < 1e-3),
where the GPU's choice must still be a valid top-k / argmax; fp32 outputs must
satisfy max|gpu - ref| <= 1e-2 * max|ref| per tensor.
"""
import numpy as np
import pytest
import torch

import moe_speculative_verify_amd as mv
import oracle
import synth
from gpu_util import (REL_TOL, TIE_BAND, assert_close, check_selection, check_tie_rows,
                      compare_route, device_layer, oracle_ffn_from_device, to_dev, to_host_bits)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    mv.lib()   # fails loudly when the HIP library is missing
    yield
    torch.cuda.synchronize()


def say(*a):
    print("CASE", *a, flush=True)


def host_case(M, H, E, I, seed, bias_alpha=None):
    x = synth.activations(M, H, seed=seed)
    w = synth.layer_weights(H, E, I, seed=synth.WEIGHT_SEED + seed) if I else dict(
        router=synth.normal_bf16((E, H), synth.WEIGHT_STD, synth.WEIGHT_SEED + seed, 0, 0))
    bias = None if bias_alpha is None else synth.zipf_bias(E, bias_alpha)
    return x, w, bias


def run_route(x, wr, bias, k, want_logits=True):
    b = None if bias is None else torch.from_numpy(bias).cuda()
    idx, w, lg = mv.moe_route(to_dev(x) if isinstance(x, np.ndarray) else x,
                              to_dev(wr) if isinstance(wr, np.ndarray) else wr, k, b,
                              want_logits=True)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), w.cpu().numpy(), lg.cpu().numpy()


# ----------------------------------------------------------------- router

ROUTE_CASES = [
    # M, H, E, k, bias alpha
    (1, 256, 16, 2, None),       # tiny layer's router
    (3, 264, 20, 4, 1.0),        # ragged: 33 chunks per row, E not a multiple of 64
    (16, 256, 16, 16, None),     # k = E
    (1, 8, 1, 1, None),          # smallest shape
    (6, 2560, 512, 8, None),     # router gate, verify width 6
    (6, 2560, 512, 8, 1.0),      # with Zipf bias
    (16, 2560, 512, 8, 1.0),     # block-16 verify
    (5, 4096, 1024, 16, 0.5),    # largest E and k
    (8, 8192, 256, 8, None),     # widest hidden state staged in LDS
    (16, 8192, 1024, 16, 0.5),   # hidden states too large for LDS: read from the caches
    (9, 2560, 512, 8, None),     # one token past the packed launch shape
    (12, 520, 100, 6, 1.0),      # ragged: 65 chunks per row, 100 experts
]


@pytest.mark.parametrize("M,H,E,k,alpha", ROUTE_CASES)
def test_route_matches_oracle(M, H, E, k, alpha):
    say("route", M, H, E, k, alpha)
    x, w, bias = host_case(M, H, E, None, seed=100 + M + E, bias_alpha=alpha)
    gi, gw, gl = run_route(x, w["router"], bias, k)
    ref = oracle.route(x, w["router"], bias, k)
    compare_route(gi, gw, gl, ref, k)


def test_route_zero_input_and_planted_ties():
    say("route special cases")
    M, H, E, k = 2, 256, 16, 4
    wr = synth.normal_bf16((E, H), 0.02, 7, 1)
    gi, gw, gl = run_route(np.zeros((M, H), np.uint16), wr, None, k)
    assert np.array_equal(gi, np.tile(np.arange(k), (M, 1)))
    assert np.all(gw == np.float32(1.0 / k)) and np.all(gl == 0.0)
    # duplicated router rows tie exactly: the lower id must come first
    x = synth.activations(M, H, seed=8)
    ref = oracle.route(x, wr, None, k)
    top = ref["idx"][:, 0]
    wr2 = wr.copy()
    wr2[0] = wr[top[0]]
    wr2[15] = wr[top[1]]
    gi, _, gl = run_route(x, wr2, None, k)
    assert gi[0, 0] == min(0, top[0]) and top[0] in gi[0, :2] and 0 in gi[0, :2]
    assert gl[0, 0] == gl[0, top[0]]
    assert gi[1, 0] == top[1] and gi[1, 1] == 15
    # exact doubling of x doubles the logits exactly and keeps the ids
    x2 = synth.bf16_bits(synth.bf16_to_f32(x) * 2)
    gi_a, _, gl_a = run_route(x, wr, None, k)
    gi_b, _, gl_b = run_route(x2, wr, None, k)
    assert np.array_equal(gi_a, gi_b) and np.array_equal(gl_b, 2 * gl_a)


@pytest.mark.parametrize("E,k,M", [(512, 8, 1), (1024, 16, 1), (200, 8, 1), (512, 8, 12)])
def test_route_planted_ties_full_width(E, k, M):
    """Zero hidden states make the logits equal to the bias exactly; a bias
    with few distinct values plants ties inside a lane (ids e and e + 64) and
    across lanes. Order is value descending, then id ascending. M = 12 runs
    the launch shape for more than eight tokens, every row the same."""
    say("route planted ties", E, k, M)
    H = 2560
    wr = synth.normal_bf16((E, H), 0.02, 9, E)
    bias = np.stack([((np.arange(E) * (31 + 6 * t)) % (5 + t)).astype(np.float32)
                     for t in range(3)])
    for t in range(3):
        gi, gw, gl = run_route(np.zeros((M, H), np.uint16), wr, bias[t].copy(), k)
        order = np.lexsort((np.arange(E), -bias[t].astype(np.float64)))[:k]
        ref = oracle.route(np.zeros((1, H), np.uint16), wr, bias[t].copy(), k)
        assert np.array_equal(ref["idx"][0], order)
        for r in range(M):
            assert np.array_equal(gi[r], order), (t, r, gi[r], order)
            assert np.array_equal(gl[r], bias[t])
            assert_close(gw[r], ref["w"][0], "topk_w")


# ----------------------------------------------------------- expert FFN

def _ffn_host(M, H, I, E, k, seed, skew=0.0):
    x = synth.activations(M, H, seed=seed)
    w = synth.layer_weights(H, E, I, seed=synth.WEIGHT_SEED + seed)
    idx, tw = synth.random_routing(M, E, k, seed, skew)
    return x, w, idx, tw


FFN_CASES = [
    # M, H, I, E, k
    (1, 256, 128, 16, 2),        # tiny layer
    (3, 264, 136, 20, 4),        # ragged chunk counts
    (16, 256, 128, 16, 16),      # every token uses every expert
    (2, 8, 8, 3, 2),             # smallest shape
    (7, 512, 1032, 40, 3),       # I not a multiple of the 512-element lane stride
    (1, 1032, 256, 12, 3),       # one token, x in registers, a partial last chunk column
    (1, 3072, 256, 16, 4),       # one token, two K blocks per unit: x staged in LDS
    # the up kernel deals its units in periods of 10 rounds of 256 plus 128
    # units for the even-numbered workgroups (2688); a partial last period
    # deals its rounds first, then the rest to the even ones:
    (1, 256, 1304, 8, 2),        # 2608 units: 48 past the partial period's rounds
    (1, 3072, 3992, 8, 2),       # 7984 = 2 periods + 2608, two K blocks per unit
]


@pytest.mark.parametrize("M,H,I,E,k", FFN_CASES)
def test_expert_ffn_matches_oracle(M, H, I, E, k):
    say("expert_ffn", M, H, I, E, k)
    x, w, idx, tw = _ffn_host(M, H, I, E, k, seed=200 + M + I)
    dw = {key: to_dev(w[key]) for key in ("gate", "up", "down")}
    out = mv.moe_expert_ffn(to_dev(x), torch.from_numpy(idx).cuda(),
                            torch.from_numpy(tw).cuda(), dw["gate"], dw["up"], dw["down"])
    got = out.cpu().numpy()
    ref = oracle.expert_ffn(x, idx, tw.astype(np.float64), w["gate"], w["up"], w["down"])
    assert_close(got, ref, "out")


@pytest.fixture(scope="module")
def full_layer():
    say("generating full-size layer weights on the device")
    return device_layer(2560, 512, 1024)


@pytest.mark.parametrize("M,skew", [(1, 0.0), (6, 0.0), (16, 0.0), (16, 1.0)])
def test_expert_ffn_full_size(full_layer, M, skew):
    say("expert_ffn full size", M, skew)
    k = 8
    x = synth.activations(M, 2560, seed=300 + M)
    idx, tw = synth.random_routing(M, 512, k, 300 + M, skew)
    out = mv.moe_expert_ffn(to_dev(x), torch.from_numpy(idx).cuda(),
                            torch.from_numpy(tw).cuda(), full_layer["gate"],
                            full_layer["up"], full_layer["down"])
    got = out.cpu().numpy()
    ref = oracle_ffn_from_device(x, idx, tw.astype(np.float64), full_layer)
    assert_close(got, ref, "out")


LIMIT_CASES = [
    # M, H, I, E, k, routing skew
    (5, 4096, 2048, 8, 4, 0.0),      # widest H of the down GEMV (16 rows per workgroup); 2 K blocks up
    (16, 512, 256, 1024, 16, 0.0),   # most experts and slots: 256 pairs over 1024 experts
    (2, 256, 8192, 8, 2, 0.0),       # largest I: 16 K blocks of every down row
    (16, 1024, 512, 64, 8, 1.0),     # skewed routing: hot experts with up to 16 pairs
]


@pytest.mark.parametrize("M,H,I,E,k,skew", LIMIT_CASES)
def test_expert_ffn_limits(M, H, I, E, k, skew):
    say("expert_ffn limits", M, H, I, E, k, skew)
    dw = device_layer(H, E, I, seed=synth.WEIGHT_SEED + H + I)
    x = synth.activations(M, H, seed=500 + M + I)
    idx, tw = synth.random_routing(M, E, k, 500 + E, skew)
    out = mv.moe_expert_ffn(to_dev(x), torch.from_numpy(idx).cuda(), torch.from_numpy(tw).cuda(),
                            dw["gate"], dw["up"], dw["down"])
    got = out.cpu().numpy()
    ref = oracle_ffn_from_device(x, idx, tw.astype(np.float64), dw)
    assert_close(got, ref, "out")
    del dw


@pytest.mark.parametrize("M", [3, 6])
def test_expert_ffn_identical_tokens_share_experts(full_layer, M):
    """M identical tokens route identically: every row equals the M=1 row,
    bit for bit (with bf16 weights every column block runs on the GEMV
    path however many pairs it holds)."""
    say("expert_ffn identical tokens", M)
    x1 = synth.activations(1, 2560, seed=41)
    idx1, tw1 = synth.random_routing(1, 512, 8, 41)
    x = np.repeat(x1, M, axis=0)
    idx = np.repeat(idx1, M, axis=0)
    tw = np.repeat(tw1, M, axis=0)
    a = mv.moe_expert_ffn(to_dev(x1), torch.from_numpy(idx1).cuda(), torch.from_numpy(tw1).cuda(),
                          full_layer["gate"], full_layer["up"], full_layer["down"]).cpu().numpy()
    b = mv.moe_expert_ffn(to_dev(x), torch.from_numpy(idx).cuda(), torch.from_numpy(tw).cuda(),
                          full_layer["gate"], full_layer["up"], full_layer["down"]).cpu().numpy()
    for t in range(M):
        assert np.array_equal(b[t], a[0])


def test_expert_ffn_invalid_ids_contribute_nothing():
    say("expert_ffn invalid ids")
    M, H, I, E, k = 3, 256, 128, 16, 4
    x, w, idx, tw = _ffn_host(M, H, I, E, k, seed=51)
    dw = {key: to_dev(w[key]) for key in ("gate", "up", "down")}
    bad = idx.copy()
    bad[0, 1] = -1
    bad[2, 3] = E + 5
    out = mv.moe_expert_ffn(to_dev(x), torch.from_numpy(bad).cuda(), torch.from_numpy(tw).cuda(),
                            dw["gate"], dw["up"], dw["down"]).cpu().numpy()
    tw0 = tw.astype(np.float64).copy()
    tw0[0, 1] = 0.0
    tw0[2, 3] = 0.0
    fixed = np.where(bad < 0, 0, np.where(bad >= E, 0, bad)).astype(np.int32)
    ref = oracle.expert_ffn(x, fixed, tw0, w["gate"], w["up"], w["down"])
    assert_close(out, ref, "out")


def test_expert_ffn_single_expert_scaling():
    """k = 1, weight 1: doubling W_down (exact in bf16) doubles out exactly."""
    say("expert_ffn scaling")
    M, H, I, E = 4, 512, 256, 8
    x, w, _, _ = _ffn_host(M, H, I, E, 1, seed=61)
    idx = np.array([[3], [3], [5], [0]], np.int32)
    tw = np.ones((M, 1), np.float32)
    dw = {key: to_dev(w[key]) for key in ("gate", "up", "down")}
    a = mv.moe_expert_ffn(to_dev(x), torch.from_numpy(idx).cuda(), torch.from_numpy(tw).cuda(),
                          dw["gate"], dw["up"], dw["down"]).cpu().numpy()
    d2 = to_dev(synth.bf16_bits(synth.bf16_to_f32(w["down"]) * 2))
    b = mv.moe_expert_ffn(to_dev(x), torch.from_numpy(idx).cuda(), torch.from_numpy(tw).cuda(),
                          dw["gate"], dw["up"], d2).cpu().numpy()
    assert np.array_equal(b, 2 * a)
    ref = oracle.expert_ffn(x, idx, tw.astype(np.float64), w["gate"], w["up"], w["down"])
    assert_close(a, ref, "out")


def test_layer_expert_relabeling():
    """Renaming the experts (router rows, weight slabs and bias entries moved
    by one permutation) renames the selected ids and leaves the weights and
    the output bitwise unchanged: no result depends on an expert's id or
    position beyond the lowest-id tie rule."""
    say("layer expert relabeling")
    M, H, I, E, k = 6, 512, 256, 64, 4
    x, w, bias = host_case(M, H, E, I, seed=71, bias_alpha=1.0)
    perm = synth.rng(72).permutation(E)      # expert e is renamed perm[e]
    wp, bp = {}, np.empty_like(bias)
    for key, v in w.items():
        wp[key] = np.empty_like(v)
        wp[key][perm] = v
    bp[perm] = bias
    gi, gw, go = _layer_gpu(x, {key: to_dev(v) for key, v in w.items()}, bias, k)
    pi, pw, po = _layer_gpu(x, {key: to_dev(v) for key, v in wp.items()}, bp, k)
    ref = oracle.route(x, w["router"], bias, k)
    tied = [t for t in range(M) if ref["gap_sel"][t] < TIE_BAND or ref["gap_order"][t] < TIE_BAND]
    for t in range(M):
        if t in tied:           # the lowest-id rule may order a tie differently
            continue
        assert np.array_equal(pi[t], perm[gi[t]]), (t, pi[t], perm[gi[t]])
        assert np.array_equal(pw[t], gw[t])
        assert np.array_equal(po[t], go[t])


# ------------------------------------------------------------- full layer

def _layer_gpu(x, w, bias, k):
    b = None if bias is None else torch.from_numpy(bias).cuda()
    idx, tw, out = mv.moe_layer(to_dev(x), w["router"], w["gate"], w["up"], w["down"], k, b)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), tw.cpu().numpy(), out.cpu().numpy()


def test_layer_tiny():
    say("layer tiny")
    cfg = synth.WORKLOADS["tiny"]
    x, w, _ = host_case(cfg["M"], cfg["H"], cfg["E"], cfg["I"], seed=0)
    dw = {key: to_dev(v) for key, v in w.items()}
    gi, gw, go = _layer_gpu(x, dw, None, cfg["k"])
    ref = oracle.route(x, w["router"], None, cfg["k"])
    same = compare_route(gi, gw, None, ref, cfg["k"])
    out = oracle.expert_ffn(x, ref["idx"], ref["w"], w["gate"], w["up"], w["down"])
    assert_close(go[same], out[same], "out")
    check_tie_rows(x, gi, gw, go, ref, lambda xr, ids, tw: oracle.expert_ffn(
        xr, ids, tw, w["gate"], w["up"], w["down"]))


@pytest.mark.parametrize("M,alpha", [(1, None), (1, 1.0), (6, None), (6, 1.0), (16, 1.0),
                                     (16, 0.0)])
def test_layer_full_size(full_layer, M, alpha):
    say("layer full size", M, alpha)
    k = 8
    x = synth.activations(M, 2560, seed=400 + M)
    bias = None if alpha is None else synth.zipf_bias(512, alpha)
    gi, gw, go = _layer_gpu(x, full_layer, bias, k)
    wr = to_host_bits(full_layer["router"])
    ref = oracle.route(x, wr, bias, k)
    same = compare_route(gi, gw, None, ref, k)
    assert len(same) >= M - 1, "more than one near-tie in a handful of tokens"
    out = oracle_ffn_from_device(x, ref["idx"], ref["w"], full_layer)
    assert_close(go[same], out[same], "out")
    check_tie_rows(x, gi, gw, go, ref,
                   lambda xr, ids, w: oracle_ffn_from_device(xr, ids, w, full_layer))


@pytest.mark.parametrize("M,H,E,I,k,alpha", [
    (1, 2560, 512, 1024, 8, None),   # four slices of the hidden dimension, one token
    (6, 2560, 512, 1024, 8, 1.0),    # the verify width, with the router bias
    (16, 2560, 512, 1024, 8, None),  # 16 tokens: two tokens per selecting wavefront
    (3, 264, 20, 136, 4, 1.0),       # one slice, ragged E (keys past E absent)
    (12, 520, 100, 64, 6, None),     # one slice, 12 tokens
    (9, 1024, 384, 256, 16, 0.5),    # k = 16
])
def test_layer_selection_in_up_kernel_equals_route_then_ffn(M, H, E, I, k, alpha):
    """With at most 512 experts moe_layer selects inside the up kernel from
    the router kernel's partial logits; its ids, weights and output equal
    moe_route followed by moe_expert_ffn bit for bit."""
    say("layer selection in the up kernel", M, H, E, I, k, alpha)
    dw = device_layer(H, E, I, seed=synth.WEIGHT_SEED + 7 * H + E)
    x = to_dev(synth.activations(M, H, seed=1700 + M))
    b = None if alpha is None else torch.from_numpy(synth.zipf_bias(E, alpha)).cuda()
    li, lw, lo = mv.moe_layer(x, dw["router"], dw["gate"], dw["up"], dw["down"], k, b)
    ri, rw = mv.moe_route(x, dw["router"], k, b)
    ro = mv.moe_expert_ffn(x, ri, rw, dw["gate"], dw["up"], dw["down"])
    torch.cuda.synchronize()
    assert torch.equal(li, ri) and torch.equal(lw, rw) and torch.equal(lo, ro)


def test_layer_more_than_512_experts():
    """Above 512 experts the router kernel selects (the up kernel's prologue
    holds 8 logits per lane): moe_layer against the oracle at E = 1024."""
    M, H, E, I, k = 5, 256, 1024, 128, 16
    say("layer E=1024", M, H, E, I, k)
    x, w, bias = host_case(M, H, E, I, seed=1800, bias_alpha=0.5)
    gi, gw, go = _layer_gpu(x, {key: to_dev(v) for key, v in w.items()}, bias, k)
    ref = oracle.route(x, w["router"], bias, k)
    same = compare_route(gi, gw, None, ref, k)
    out = oracle.expert_ffn(x, ref["idx"], ref["w"], w["gate"], w["up"], w["down"])
    assert_close(go[same], out[same], "out")
    check_tie_rows(x, gi, gw, go, ref, lambda xr, ids, tw: oracle.expert_ffn(
        xr, ids, tw, w["gate"], w["up"], w["down"]))


# ---------------------------------------------------------------- lm_head

def _lm_gpu(h, wl):
    am, ml = mv.lmhead_argmax(to_dev(h), wl if isinstance(wl, torch.Tensor) else to_dev(wl),
                              want_max=True)
    torch.cuda.synchronize()
    return am.cpu().numpy(), ml.cpu().numpy()


def _compare_lm(am, ml, h, wl_bits, ref):
    M = h.shape[0]
    for t in range(M):
        if am[t] != ref["tok"][t]:
            assert ref["gap"][t] < TIE_BAND, f"token {t}: {am[t]} != {ref['tok'][t]}"
            zt = synth.bf16_to_f32(h[t]).astype(np.float64) @ \
                synth.bf16_to_f32(wl_bits[am[t]]).astype(np.float64)
            assert zt >= ref["zmax"][t] - TIE_BAND
    assert_close(ml, ref["zmax"], "max_logit")


# (6, 2560, 30272): 1892 tiles of 16 rows over 256 workgroups, 8 or 7 per
# workgroup (wavefronts with 2 or 1 tiles); (4, 1024, 22560): 1410 tiles, 6
# or 5 per workgroup
@pytest.mark.parametrize("M,H,V", [(1, 256, 1000), (3, 264, 777), (16, 256, 4099),
                                   (6, 2560, 65), (2, 8, 1), (6, 2560, 30272),
                                   (4, 1024, 22560)])
def test_lmhead_matches_oracle(M, H, V):
    say("lmhead", M, H, V)
    h = synth.activations(M, H, seed=500 + V)
    wl = synth.normal_bf16((V, H), synth.WEIGHT_STD, synth.WEIGHT_SEED, 9, V)
    am, ml = _lm_gpu(h, wl)
    _compare_lm(am, ml, h, wl, oracle.lmhead(h, wl))


def test_lmhead_full_size():
    say("lmhead full size 6 x 2560 x 157184")
    M, H, V = 6, 2560, 157184
    h = synth.activations(M, H, seed=601)
    wl = synth.device_normal_bf16((V, H), synth.WEIGHT_STD, synth.WEIGHT_SEED, 0,
                                  synth.KIND["lm_head"])
    # planted winners: the last row for token 0, a row equal to h for token 1,
    # and two equal copies for token 2 (lower id must win)
    hd = to_dev(h)
    wl[V - 1] = hd[0] * 4
    wl[1234] = hd[1] * 4
    wl[90000] = hd[2] * 4
    wl[777] = hd[2] * 4
    am, ml = _lm_gpu(h, wl)
    assert am[0] == V - 1 and am[1] == 1234 and am[2] == 777
    wl_bits = to_host_bits(wl)
    _compare_lm(am, ml, h, wl_bits, oracle.lmhead(h, wl_bits))


@pytest.mark.parametrize("M,H,V,fp8", [(6, 2560, 5000, False), (16, 256, 4099, False),
                                        (1, 264, 100, False), (6, 1040, 3001, True)])
def test_lmhead_phases_equal_the_combined_call(M, H, V, fp8):
    """lmhead_partial_keys then lmhead_merge_keys gives bitwise what
    lmhead_greedy_verify (and lmhead_argmax, without tokens) gives."""
    say("lmhead phases", M, H, V, fp8)
    h = to_dev(synth.activations(M, H, seed=800 + M))
    if fp8:
        q, sc = synth.fp8_rows((V, H), synth.WEIGHT_STD, synth.WEIGHT_SEED, 801, V)
        w, sc = torch.from_numpy(q).cuda(), torch.from_numpy(sc).cuda()
    else:
        w, sc = to_dev(synth.normal_bf16((V, H), 0.02, 802, V)), None
    chain = torch.from_numpy(np.random.default_rng(803).integers(0, V, size=M).astype(np.int32)).cuda()
    if fp8:
        am0, acc0, ml0 = mv.lmhead_greedy_verify_fp8(h, w, sc, chain, want_max=True)
    else:
        am0, acc0, ml0 = mv.lmhead_greedy_verify(h, w, chain, want_max=True)
    ws = torch.zeros(mv.lmhead_argmax_workspace_bytes(M, V), dtype=torch.uint8, device="cuda")
    mv.lmhead_partial_keys(h, w, ws, w_scale=sc)
    am1, acc1, ml1 = mv.lmhead_merge_keys(M, V, ws, tokens=chain, want_max=True)
    am2 = mv.lmhead_merge_keys(M, V, ws)
    torch.cuda.synchronize()
    assert torch.equal(am0, am1) and torch.equal(acc0, acc1) and torch.equal(ml0, ml1)
    assert torch.equal(am0, am2)


def test_lmhead_zero_hidden():
    say("lmhead zero hidden")
    wl = synth.normal_bf16((300, 64), 0.02, 3, 3)
    am, ml = _lm_gpu(np.zeros((2, 64), np.uint16), wl)
    assert am.tolist() == [0, 0] and np.all(ml == 0.0)


def test_lmhead_all_minus_inf():
    """Every logit overflows to -inf in fp32 (finite bf16 inputs whose
    products exceed the fp32 range): the argmax is row 0, as the oracle's
    first-index rule on its fp32-rounded logits gives, and a row whose logit
    is finite wins over the -inf rows."""
    say("lmhead all -inf")
    M, H, V = 3, 256, 4099
    big = synth.bf16_bits(np.float32([2.0 ** 100]))[0]
    h = np.zeros((M, H), np.uint16)
    h[:, 0] = big
    wl = np.zeros((V, H), np.uint16)
    wl[:, 0] = synth.bf16_bits(np.float32([-(2.0 ** 100)]))[0]
    am, ml = _lm_gpu(h, wl)
    ref = oracle.lmhead(h, wl)
    assert am.tolist() == [0] * M == ref["tok"].tolist()
    assert np.all(np.isneginf(ml))
    wl[2500, 0] = synth.bf16_bits(np.float32([2.0 ** -10]))[0]
    am, ml = _lm_gpu(h, wl)
    assert am.tolist() == [2500] * M == oracle.lmhead(h, wl)["tok"].tolist()
    assert np.all(ml == np.float32(2.0 ** 90))


def test_side_stream_matches_default_stream(full_layer):
    """moe_layer and lmhead_greedy_verify enqueued on a side stream (their
    pooled workspaces allocated and zero-filled on that stream) give the
    default stream's results bit for bit."""
    say("side stream")
    k, M, V = 8, 6, 20000
    fw = full_layer
    x = to_dev(synth.activations(M, 2560, seed=1300))
    h = to_dev(synth.activations(M, 2560, seed=1301))
    wl = to_dev(synth.normal_bf16((V, 2560), synth.WEIGHT_STD, 1302, 0))
    chain = torch.zeros(M, dtype=torch.int32, device="cuda")
    a = mv.moe_layer(x, fw["router"], fw["gate"], fw["up"], fw["down"], k)
    la = mv.lmhead_greedy_verify(h, wl, chain)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        b = mv.moe_layer(x, fw["router"], fw["gate"], fw["up"], fw["down"], k, stream=side)
        lb = mv.lmhead_greedy_verify(h, wl, chain, stream=side)
    torch.cuda.synchronize()
    for ta, tb in zip(a + la, b + lb):
        assert torch.equal(ta, tb)


# --------------------------------------------------- greedy verify verdict

def _verify_gpu(h, wl, chain):
    am, acc, ml = mv.lmhead_greedy_verify(
        to_dev(h), wl if isinstance(wl, torch.Tensor) else to_dev(wl),
        torch.from_numpy(np.ascontiguousarray(chain, np.int32)).to("cuda"), want_max=True)
    torch.cuda.synchronize()
    return am.cpu().numpy(), acc.cpu().numpy(), ml.cpu().numpy()


def _chains(tok, V, rng):
    """Chains against the target tokens tok: followed throughout, rejected at
    each position j (later candidates still follow), and one random chain."""
    M = tok.shape[0]
    full = np.concatenate([[rng.integers(0, V)], tok[:-1]]).astype(np.int32)
    out = [full]
    for j in range(1, M):
        c = full.copy()
        c[j] = (tok[j - 1] + 1) % max(V, 2)
        out.append(c)
    out.append(rng.integers(0, V, size=M).astype(np.int32))
    return out


@pytest.mark.parametrize("M,H,V", [(6, 2560, 4099), (1, 256, 1000), (16, 256, 4099),
                                   (5, 264, 777), (2, 8, 1)])
def test_greedy_verify_matches_oracle(M, H, V):
    say("greedy verify", M, H, V)
    h = synth.activations(M, H, seed=1500 + V)
    wl = synth.normal_bf16((V, H), synth.WEIGHT_STD, synth.WEIGHT_SEED, 19, V)
    ref = oracle.lmhead(h, wl)
    am0, ml0 = _lm_gpu(h, wl)
    rng = np.random.default_rng(M * 1000 + V)
    for chain in _chains(ref["tok"], V, rng):
        am, acc, ml = _verify_gpu(h, wl, chain)
        # the argmax is lmhead_argmax's, bit for bit, and matches the oracle
        assert np.array_equal(am, am0) and np.array_equal(ml, ml0)
        _compare_lm(am, ml, h, wl, ref)
        # the verdict is exact given the kernel's tokens, and equals the
        # oracle's verdict on the oracle's tokens whenever those agree
        assert tuple(acc) == oracle.greedy_verdict(chain, am)
        if np.array_equal(am, ref["tok"]):
            assert tuple(acc) == oracle.greedy_verdict(chain, ref["tok"])


def test_greedy_verify_full_size():
    """Full lm_head (157184 x 2560, M = 6) with planted winners, so every
    target token is known exactly: the chain is accepted up to a planted
    rejection at position 3."""
    say("greedy verify full size 6 x 2560 x 157184")
    M, H, V = 6, 2560, 157184
    h = synth.activations(M, H, seed=1601)
    wl = synth.device_normal_bf16((V, H), synth.WEIGHT_STD, synth.WEIGHT_SEED, 0,
                                  synth.KIND["lm_head"])
    hd = to_dev(h)
    rows = [V - 1, 1234, 777, 90001, 5, 150000]
    for t, r in enumerate(rows):
        wl[r] = hd[t] * 4
    chain = np.array([42, rows[0], rows[1], rows[2] + 1, rows[3], rows[4]], np.int32)
    am, acc, ml = _verify_gpu(h, wl, chain)
    assert am.tolist() == rows
    assert acc.tolist() == [3, rows[2]]
    wl_bits = to_host_bits(wl)
    _compare_lm(am, ml, h, wl_bits, oracle.lmhead(h, wl_bits))
    assert tuple(acc) == oracle.greedy_verdict(chain, np.array(rows, np.int32))
    chain_all = np.array([42] + rows[:5], np.int32)
    _, acc2, _ = _verify_gpu(h, wl, chain_all)
    assert acc2.tolist() == [6, rows[5]]


# --------------------------------------------- determinism and invariance

def test_determinism_and_batch_invariance(full_layer):
    """Two runs are bitwise equal, and each token's results equal the same
    token run alone (no float atomics; per-token order fixed)."""
    say("determinism / batch invariance")
    M, k = 6, 8
    x = synth.activations(M, 2560, seed=701)
    runs = [_layer_gpu(x, full_layer, None, k) for _ in range(2)]
    for a, b in zip(runs[0], runs[1]):
        assert np.array_equal(a, b)
    gi, gw, go = runs[0]
    for t in (0, 3, 5):
        gi1, gw1, go1 = _layer_gpu(x[t:t + 1], full_layer, None, k)
        assert np.array_equal(gi1[0], gi[t])
        assert np.array_equal(gw1[0], gw[t])
        assert np.array_equal(go1[0], go[t])
    wl = synth.normal_bf16((5000, 2560), 0.02, 4, 4)
    am, ml = _lm_gpu(x, wl)
    for t in (1, 4):
        am1, ml1 = _lm_gpu(x[t:t + 1], wl)
        assert am1[0] == am[t] and ml1[0] == ml[t]


def test_batch_invariance_across_regimes(full_layer):
    """At M = 16 the router sums each logit over 16-row tiles and the down
    projection runs on the MFMA kernel; alone (M = 1) a token takes the
    8-row router tiles and the GEMV down kernel. Both sum in other orders, so
    across these regimes a token's results agree within rounding, not bit
    for bit: the same ids (unless the oracle flags a near-tie), weights and
    output within the fp32 tolerance of each other and of the oracle."""
    say("batch invariance across the router and down-kernel regimes")
    M, k = 16, 8
    x = synth.activations(M, 2560, seed=703)
    gi, gw, go = _layer_gpu(x, full_layer, None, k)
    ref = oracle.route(x, to_host_bits(full_layer["router"]), None, k)
    same16 = compare_route(gi, gw, None, ref, k)
    for t in (0, 7, 15):
        gi1, gw1, go1 = _layer_gpu(x[t:t + 1], full_layer, None, k)
        if t not in same16 or not np.array_equal(gi1[0], ref["idx"][t]):
            continue                                  # a near-tie (checked above)
        assert np.array_equal(gi1[0], gi[t])
        assert_close(gw[t], gw1[0], f"token {t}: weights at M=16 against alone")
        assert_close(go[t], go1[0], f"token {t}: output at M=16 against alone")
        out = oracle_ffn_from_device(x[t:t + 1], ref["idx"][t:t + 1], ref["w"][t:t + 1],
                                     full_layer)
        assert_close(go[t:t + 1], out, f"token {t}: output at M=16 against the oracle")


def test_workspace_shared_by_every_entry_point(full_layer):
    """One workspace serves moe_layer, lmhead_argmax, moe_route and
    lmhead_greedy_verify in turn with no clearing in between (whatever one
    call leaves past the header must not change the next call's results):
    every result equals the same call on a fresh zero-filled workspace, and
    the header is zero after every call."""
    say("workspace shared by every entry point")
    k, H, E, I = 8, 2560, 512, 1024
    M, V = 6, 20000
    nbytes = max(mv.moe_layer_workspace_bytes(16, H, I, E, k),
                 mv.lmhead_argmax_workspace_bytes(16, V), mv.moe_route_workspace_bytes(16, E))
    shared = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    fw = full_layer
    x = to_dev(synth.activations(M, H, seed=1200))
    h = to_dev(synth.activations(M, H, seed=1201))
    # small lm_head logits (|z| ~ 0.03): a key left over from another call
    # (route logits ~ N(0, 1)) would win any argmax that read it
    wl = to_dev(synth.normal_bf16((V, H), 0.0005, 1202, 0))

    def fresh():
        return torch.zeros(nbytes, dtype=torch.uint8, device="cuda")

    chain = torch.zeros(M, dtype=torch.int32, device="cuda")
    calls = [
        lambda ws: mv.moe_layer(x, fw["router"], fw["gate"], fw["up"], fw["down"], k,
                                workspace=ws),
        lambda ws: mv.lmhead_argmax(h, wl, want_max=True, workspace=ws),
        lambda ws: mv.moe_route(x, fw["router"], k, want_logits=True, workspace=ws),
        lambda ws: mv.lmhead_greedy_verify(h, wl, chain, workspace=ws),
        lambda ws: mv.moe_layer(x, fw["router"], fw["gate"], fw["up"], fw["down"], k,
                                workspace=ws),
    ]
    for i, call in enumerate(calls):
        a = call(fresh())
        b = call(shared)
        torch.cuda.synchronize()
        for ta, tb in zip(a, b):
            assert torch.equal(ta, tb), (i, "result")
        assert int(shared[:4096].count_nonzero()) == 0, (i, "header")


def test_workspace_reuse_across_shapes():
    """Counters left at zero: calls of different shapes reuse one workspace."""
    say("workspace reuse")
    for (M, H, E, k) in [(6, 2560, 512, 8), (1, 256, 16, 2), (16, 512, 64, 4), (6, 2560, 512, 8)]:
        x, w, _ = host_case(M, H, E, None, seed=800 + M)
        gi, gw, gl = run_route(x, w["router"], None, k)
        compare_route(gi, gw, gl, oracle.route(x, w["router"], None, k), k)
    for (M, V) in [(6, 20000), (1, 100), (6, 20000)]:
        h = synth.activations(M, 256, seed=900 + M)
        wl = synth.normal_bf16((V, 256), 0.02, 5, V)
        am, ml = _lm_gpu(h, wl)
        _compare_lm(am, ml, h, wl, oracle.lmhead(h, wl))


def test_layer_workspace_shared_across_M(full_layer):
    """One workspace serves moe_layer at M = 6, 1, 16, 6 in turn, with
    moe_expert_ffn calls in between: every result equals the same call on a
    fresh zero-filled workspace, and the 4 KB header of counters is
    zero after every call (the header sits at fixed offsets for every
    shape)."""
    say("workspace shared across M")
    k, H, I, E = 8, 2560, 1024, 512
    nbytes = max(mv.moe_layer_workspace_bytes(M, H, I, E, k) for M in (1, 6, 16))
    shared = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    fw = full_layer
    for i, M in enumerate((6, 1, 16, 6)):
        x = to_dev(synth.activations(M, H, seed=1000 + i))
        fresh = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
        a = mv.moe_layer(x, fw["router"], fw["gate"], fw["up"], fw["down"], k, workspace=fresh)
        b = mv.moe_layer(x, fw["router"], fw["gate"], fw["up"], fw["down"], k, workspace=shared)
        torch.cuda.synchronize()
        for ta, tb in zip(a, b):
            assert torch.equal(ta, tb), (M, "layer")
        assert int(shared[:4096].count_nonzero()) == 0, (M, "header after moe_layer")
        # the FFN alone on the same workspace, routed by the layer's ids
        c = mv.moe_expert_ffn(x, a[0], a[1], fw["gate"], fw["up"], fw["down"], workspace=shared)
        torch.cuda.synchronize()
        assert torch.equal(c, a[2]), (M, "ffn")
        assert int(shared[:4096].count_nonzero()) == 0, (M, "header after moe_expert_ffn")


def test_hbm_read_probe_checksum():
    """The streaming-read probe reads every word once: the XOR of its
    per-workgroup checksums equals the XOR of the buffer's 32-bit words, with
    a ragged tail past the last full grid-stride sweep."""
    nbytes = 64 * 2**20 + 48
    say("hbm read probe", nbytes)
    words = synth.rng(90).integers(0, 2**32, size=nbytes // 4, dtype=np.uint64).astype(np.uint32)
    buf = torch.from_numpy(words.view(np.int32)).cuda()
    cs = mv.moe_hbm_read_probe(buf)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(cs.cpu().numpy().view(np.uint32))
    assert got == np.bitwise_xor.reduce(words)
