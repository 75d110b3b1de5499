"""GPU parity of the router chain's norm (moe_route_rmsnorm,
moe_layer_rmsnorm) against the fp64 CPU oracle.

The normalised rows are bf16: the kernel scales in fp32 and rounds once, the
oracle rounds the fp64 value, so an element whose value lies within fp32
rounding of a bf16 midpoint may land one bf16 step apart. The test allows
that for at most 0.2% of the elements and never more than one step. The
route and the layer are then held to the usual rules against the oracle run
on the oracle's own normalised rows (indices exact except at flagged
near-ties, fp32 outputs within 1e-2 * max|ref|), and, bit for bit, to the
plain moe_route / moe_layer run on the rows the kernel wrote.
"""
import numpy as np
import pytest
import torch

import moe_speculative_verify_amd as mv
import oracle
import synth
from gpu_util import (assert_close, check_tie_rows, compare_route, device_layer,
                      oracle_ffn_from_device, to_dev, to_host_bits)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    mv.lib()
    yield
    torch.cuda.synchronize()


def say(*a):
    print("CASE", *a, flush=True)


def compare_xn(gxn: np.ndarray, rxn: np.ndarray):
    """bf16 rows: at most one step apart, and rarely."""
    g = gxn.astype(np.int64)
    r = rxn.astype(np.int64)
    same_sign = (g >> 15) == (r >> 15)
    steps = np.where(same_sign, np.abs(g - r), np.where((g & 0x7FFF) + (r & 0x7FFF) <= 1, 1, 99))
    assert steps.max() <= 1, f"normalised rows differ by {steps.max()} bf16 steps"
    assert np.count_nonzero(steps) <= max(2, 0.002 * steps.size), np.count_nonzero(steps)


def run_route_norm(h, g, eps, wr, bias, k):
    b = None if bias is None else torch.from_numpy(bias).cuda()
    xn, idx, w, lg = mv.moe_route_rmsnorm(to_dev(h), to_dev(g), eps,
                                          to_dev(wr) if isinstance(wr, np.ndarray) else wr,
                                          k, b, want_logits=True)
    torch.cuda.synchronize()
    return to_host_bits(xn), idx.cpu().numpy(), w.cpu().numpy(), lg.cpu().numpy()


NORM_CASES = [
    # M, H, E, k, eps, bias alpha
    (6, 2560, 512, 8, 1e-6, None),
    (1, 256, 16, 2, 1e-5, None),
    (16, 512, 64, 4, 1e-6, 1.0),
    (16, 4096, 512, 8, 1e-6, None),
    (8, 8192, 256, 8, 0.0, None),
    (3, 264, 20, 4, 0.5, None),
    (2, 8, 3, 2, 1e-6, None),
]


@pytest.mark.parametrize("M,H,E,k,eps,alpha", NORM_CASES)
def test_route_rmsnorm_matches_oracle(M, H, E, k, eps, alpha):
    say("route_rmsnorm", M, H, E, k, eps, alpha)
    h = synth.hidden_states(M, H, seed=3000 + H)
    g = synth.norm_gain(H, layer=H)
    wr = synth.normal_bf16((E, H), synth.WEIGHT_STD, synth.WEIGHT_SEED, 31, E, H)
    bias = None if alpha is None else synth.zipf_bias(E, alpha)
    gxn, gi, gw, gl = run_route_norm(h, g, eps, wr, bias, k)
    rxn = oracle.rmsnorm(h, g, eps)
    compare_xn(gxn, rxn)
    compare_route(gi, gw, gl, oracle.route(rxn, wr, bias, k), k)
    # the gate read exactly the rows the kernel wrote
    b = None if bias is None else torch.from_numpy(bias).cuda()
    pi, pw, pl = mv.moe_route(to_dev(gxn), to_dev(wr), k, b, want_logits=True)
    torch.cuda.synchronize()
    assert np.array_equal(pi.cpu().numpy(), gi)
    assert np.array_equal(pw.cpu().numpy(), gw)
    assert np.array_equal(pl.cpu().numpy(), gl)


def test_route_rmsnorm_tie_and_constant_rows():
    """Planted rows (worked by hand, see the oracle pins): mean square plus
    eps exactly 1 and a product 1.53515625 midway between two bf16 values ->
    the even one (0x3FC4); a constant row with eps 0 -> +-1 exactly."""
    say("route_rmsnorm planted rows")
    H, E, k = 8, 16, 2
    h = synth.bf16_bits(np.array([[1.5] + [0.0] * 7, [-2.5] * 8], np.float32))
    g = synth.bf16_bits(np.array([1.0234375] + [1.0] * 7, np.float32))
    wr = synth.normal_bf16((E, H), synth.WEIGHT_STD, synth.WEIGHT_SEED, 33)
    # row 0: 2.25 / 8 = 0.28125, + eps 0.71875 = 1; row 1 with eps != 0 is
    # not exactly -1, so it gets its own call with eps = 0
    gxn, *_ = run_route_norm(h[:1], g, 0.71875, wr, None, k)
    assert gxn[0].tolist() == [0x3FC4] + [0] * 7
    one = synth.bf16_bits(np.ones(H, np.float32))
    gxn, *_ = run_route_norm(h[1:], one, 0.0, wr, None, k)
    assert np.all(gxn == 0xBF80)


@pytest.fixture(scope="module")
def full_layer():
    say("generating full-size layer weights on the device")
    return device_layer(2560, 512, 1024)


@pytest.mark.parametrize("M,alpha", [(1, None), (6, None), (16, 1.0)])
def test_layer_rmsnorm_full_size(full_layer, M, alpha):
    say("layer_rmsnorm full size", M, alpha)
    k, H, eps = 8, 2560, 1e-6
    h = synth.hidden_states(M, H, seed=3100 + M)
    g = synth.norm_gain(H)
    bias = None if alpha is None else synth.zipf_bias(512, alpha)
    b = None if bias is None else torch.from_numpy(bias).cuda()
    xn, gi, gw, go = mv.moe_layer_rmsnorm(to_dev(h), to_dev(g), eps, full_layer["router"],
                                          full_layer["gate"], full_layer["up"],
                                          full_layer["down"], k, b)
    torch.cuda.synchronize()
    gxn, gi, gw, go = to_host_bits(xn), gi.cpu().numpy(), gw.cpu().numpy(), go.cpu().numpy()
    rxn = oracle.rmsnorm(h, g, eps)
    compare_xn(gxn, rxn)
    ref = oracle.route(rxn, to_host_bits(full_layer["router"]), bias, k)
    same = compare_route(gi, gw, None, ref, k)
    assert len(same) >= M - 1, "more than one near-tie in a handful of tokens"
    out = oracle_ffn_from_device(rxn, ref["idx"], ref["w"], full_layer)
    assert_close(go[same], out[same], "out")
    check_tie_rows(rxn, gi, gw, go, ref,
                   lambda xr, ids, w: oracle_ffn_from_device(xr, ids, w, full_layer))
    # bit for bit the plain layer on the rows the kernel wrote
    pi, pw, po = mv.moe_layer(to_dev(gxn), full_layer["router"], full_layer["gate"],
                              full_layer["up"], full_layer["down"], k, b)
    torch.cuda.synchronize()
    assert np.array_equal(pi.cpu().numpy(), gi)
    assert np.array_equal(pw.cpu().numpy(), gw)
    assert np.array_equal(po.cpu().numpy(), go)
