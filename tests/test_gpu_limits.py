"""The widest rows the C ABI accepts at each verify width launch and match
the oracle: at the largest H of the header's limits table (by M) for the
expert FFN (bf16: GEMV and MFMA down kernels; fp8) and the lm_head (bf16,
fp8). Same acceptance rules as every parity test: indices exact except at
oracle-flagged near-ties, fp32 outputs within 1e-2 * max|ref|."""
import numpy as np
import pytest
import torch

import moe_speculative_verify_amd as mv
import oracle
import synth
from gpu_util import (TIE_BAND, assert_close, device_layer, oracle_ffn_from_device, to_dev)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    mv.lib()
    yield
    torch.cuda.synchronize()


def say(*a):
    print("CASE", *a, flush=True)


def u8(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.uint8)).cuda()


def f32(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda()


@pytest.mark.parametrize("M,H,I,E,k", [
    (8, 8192, 128, 8, 2),        # widest H at M <= 8: 2 K blocks of x per token in LDS
    (11, 6144, 128, 8, 2),       # widest H at M = 9..11
    (16, 4096, 128, 8, 2),       # widest H at M = 12..16, GEMV down kernel
    (16, 4096, 1024, 8, 8),      # the same with 128 pairs of I = 1024: MFMA down kernel
])
def test_expert_ffn_widest_rows(M, H, I, E, k):
    say("expert_ffn widest rows", M, H, I, E, k)
    dw = device_layer(H, E, I, seed=synth.WEIGHT_SEED + 7 * H + I)
    x = synth.activations(M, H, seed=900 + M)
    idx, tw = synth.random_routing(M, E, k, 900 + H, 0.0)
    out = mv.moe_expert_ffn(to_dev(x), torch.from_numpy(idx).cuda(), torch.from_numpy(tw).cuda(),
                            dw["gate"], dw["up"], dw["down"])
    got = out.cpu().numpy()
    ref = oracle_ffn_from_device(x, idx, tw.astype(np.float64), dw)
    assert_close(got, ref, "out")
    del dw


@pytest.mark.parametrize("M,H,I,E,k", [
    (8, 8192, 128, 8, 2),
    (14, 5120, 128, 8, 2),
    (16, 4096, 256, 8, 4),
])
def test_expert_ffn_fp8_widest_rows(M, H, I, E, k):
    say("expert_ffn fp8 widest rows", M, H, I, E, k)
    x = synth.activations(M, H, seed=910 + M)
    qg, sg = synth.fp8_rows((E, I, H), synth.WEIGHT_STD, 920 + H, 1)
    qu, su = synth.fp8_rows((E, I, H), synth.WEIGHT_STD, 920 + H, 2)
    qd, sd = synth.fp8_rows((E, H, I), synth.WEIGHT_STD, 920 + H, 3)
    idx, tw = synth.random_routing(M, E, k, 930 + M, 0.0)
    out = mv.moe_expert_ffn_fp8(to_dev(x), torch.from_numpy(idx).cuda(),
                                torch.from_numpy(tw).cuda(), u8(qg), f32(sg), u8(qu), f32(su),
                                u8(qd), f32(sd))
    torch.cuda.synchronize()
    ref = oracle.expert_ffn_fp8(x, idx, tw, qg, sg, qu, su, qd, sd)
    assert_close(out.cpu().numpy(), ref, "out")


def _compare_argmax(am, ml, ref):
    for t in range(am.shape[0]):
        if am[t] != ref["tok"][t]:
            assert ref["gap"][t] < TIE_BAND, f"token {t}: {am[t]} != {ref['tok'][t]}"
    assert_close(ml, ref["zmax"], "max_logit")


@pytest.mark.parametrize("M,H,V", [(16, 2816, 1000), (6, 7936, 777), (8, 5888, 4099),
                                   (5, 8192, 300)])
def test_lmhead_widest_rows(M, H, V):
    say("lmhead widest rows", M, H, V)
    h = synth.activations(M, H, seed=940 + M)
    wl = synth.normal_bf16((V, H), synth.WEIGHT_STD, synth.WEIGHT_SEED, 941, V)
    am, ml = mv.lmhead_argmax(to_dev(h), to_dev(wl), want_max=True)
    torch.cuda.synchronize()
    _compare_argmax(am.cpu().numpy(), ml.cpu().numpy(), oracle.lmhead(h, wl))


@pytest.mark.parametrize("M,H,V", [(16, 2560, 1000), (6, 7680, 777), (11, 4096, 513)])
def test_lmhead_fp8_widest_rows(M, H, V):
    say("lmhead fp8 widest rows", M, H, V)
    h = synth.activations(M, H, seed=950 + M)
    q, s = synth.fp8_rows((V, H), synth.WEIGHT_STD, synth.WEIGHT_SEED, 951, V)
    am, ml = mv.lmhead_argmax_fp8(to_dev(h), u8(q), f32(s), want_max=True)
    torch.cuda.synchronize()
    _compare_argmax(am.cpu().numpy(), ml.cpu().numpy(), oracle.lmhead_fp8(h, q, s))
