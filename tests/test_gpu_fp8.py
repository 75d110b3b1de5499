"""GPU parity of the fp8 (OCP E4M3 codes, fp32 scale per output row)
variants against the fp64 CPU oracle: lm_head argmax and verdict, expert FFN,
layer. Rules as everywhere: indices exact except at oracle-flagged near-ties,
fp32 outputs within 1e-2 * max|ref| per tensor. The kernels widen the codes
to bf16 in registers (exact), so the only differences from the oracle are
fp32 accumulation order and the one bf16 rounding of the SwiGLU product.
"""
import numpy as np
import pytest
import torch

import moe_speculative_verify_amd as mv
import oracle
import synth
from gpu_util import TIE_BAND, assert_close, check_tie_rows, compare_route, to_dev, to_host_bits

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


# ------------------------------------------------------------------ lm_head

def test_lmhead_fp8_decodes_every_code():
    """Token t = the unit vector e_t, one vocabulary row holding 16 codes,
    scale 1: max_logit[t] is exactly the value of code t (NaN codes left
    out), for all 254 finite codes, against the oracle's E4M3 decode."""
    say("lmhead fp8 every code")
    H = M = 16
    h = synth.bf16_bits(np.eye(M, H, dtype=np.float32))
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    o = oracle.load()
    for c0 in range(0, len(codes), 16):
        row = np.zeros((1, H), np.uint8)
        chunk = codes[c0:c0 + 16]
        row[0, :len(chunk)] = chunk
        am, ml = mv.lmhead_argmax_fp8(to_dev(h), u8(row), f32([1.0]), want_max=True)
        torch.cuda.synchronize()
        ml = ml.cpu().numpy()
        for t, c in enumerate(chunk):
            assert ml[t] == np.float32(o.e4m3_value(int(c))), (hex(c), ml[t])


def _compare_lm8(am, ml, ref):
    for t in range(am.shape[0]):
        if am[t] != ref["tok"][t]:
            assert ref["gap"][t] < TIE_BAND, f"token {t}: {am[t]} != {ref['tok'][t]}"
    assert_close(ml, ref["zmax"], "max_logit")


@pytest.mark.parametrize("M,H,V", [(1, 256, 1000), (6, 2560, 4099), (16, 512, 777), (3, 16, 5)])
def test_lmhead_fp8_matches_oracle(M, H, V):
    say("lmhead fp8", M, H, V)
    h = synth.activations(M, H, seed=5000 + V)
    q, s = synth.fp8_rows((V, H), synth.WEIGHT_STD, synth.WEIGHT_SEED, 81, V)
    am, ml = mv.lmhead_argmax_fp8(to_dev(h), u8(q), f32(s), want_max=True)
    torch.cuda.synchronize()
    ref = oracle.lmhead_fp8(h, q, s)
    _compare_lm8(am.cpu().numpy(), ml.cpu().numpy(), ref)
    # the verdict on a chain that follows the first two targets
    tok = am.cpu().numpy()
    chain = np.concatenate([[7], tok[:-1]]).astype(np.int32)
    if M > 2:
        chain[2] = (tok[1] + 1) % V
    am2, acc = mv.lmhead_greedy_verify_fp8(to_dev(h), u8(q), f32(s),
                                           torch.from_numpy(chain).cuda())
    torch.cuda.synchronize()
    assert np.array_equal(am2.cpu().numpy(), tok)
    assert tuple(acc.cpu().tolist()) == oracle.greedy_verdict(chain, tok)


def test_lmhead_fp8_full_size():
    say("lmhead fp8 full size 6 x 2560 x 157184")
    M, H, V = 6, 2560, 157184
    h = synth.activations(M, H, seed=5101)
    q, s = synth.device_fp8_rows((V, H), synth.WEIGHT_STD, synth.WEIGHT_SEED, 0, 90)
    am, ml = mv.lmhead_argmax_fp8(to_dev(h), q, s, want_max=True)
    torch.cuda.synchronize()
    ref = oracle.lmhead_fp8(h, q.cpu().numpy(), s.cpu().numpy())
    _compare_lm8(am.cpu().numpy(), ml.cpu().numpy(), ref)


# ----------------------------------------------------------------- experts

def fp8_experts_host(H, I, E, seed):
    qg, sg = synth.fp8_rows((E, I, H), synth.WEIGHT_STD, seed, 1)
    qu, su = synth.fp8_rows((E, I, H), synth.WEIGHT_STD, seed, 2)
    qd, sd = synth.fp8_rows((E, H, I), synth.WEIGHT_STD, seed, 3)
    return dict(gate=qg, s_gate=sg, up=qu, s_up=su, down=qd, s_down=sd)


def dev8(w):
    return {key: (u8(v) if v.dtype == np.uint8 else f32(v)) for key, v in w.items()}


FP8_CASES = [
    # M, H, I, E, k
    (1, 256, 128, 16, 2),
    (6, 272, 144, 20, 4),
    (9, 512, 1024, 64, 8),
    (2, 16, 16, 3, 2),
    (6, 2560, 1024, 32, 8),
    (1, 1040, 256, 12, 3),       # one token, x in registers, a partial last chunk column
    (1, 4096, 128, 8, 2),        # one token, x in registers, 4 chunk columns per lane
    (1, 5120, 128, 8, 2),        # one token, x in registers, 5 chunk columns per lane
    (2, 6144, 128, 8, 2),        # two K blocks per unit: running sums across blocks
    (10, 512, 1024, 64, 8),      # the block-16 verify widths: 80 and 128 pairs
    (16, 256, 1024, 16, 8),      # 128 pairs over 16 experts: 8 pairs per column block
    (12, 528, 1040, 40, 8),      # 96 pairs: a 16-element K tail, 8 rows in the last workgroup
    (16, 256, 2064, 32, 16),     # 256 pairs, three K blocks of codes per down row
]


@pytest.mark.parametrize("M,H,I,E,k", FP8_CASES)
def test_expert_ffn_fp8_matches_oracle(M, H, I, E, k):
    say("expert_ffn fp8", M, H, I, E, k)
    x = synth.activations(M, H, seed=5200 + I)
    w = fp8_experts_host(H, I, E, 5300 + H)
    idx, tw = synth.random_routing(M, E, k, 5400 + M, 0.0)
    d = dev8(w)
    out = mv.moe_expert_ffn_fp8(to_dev(x), torch.from_numpy(idx).cuda(),
                                torch.from_numpy(tw).cuda(), d["gate"], d["s_gate"], d["up"],
                                d["s_up"], d["down"], d["s_down"])
    torch.cuda.synchronize()
    ref = oracle.expert_ffn_fp8(x, idx, tw, w["gate"], w["s_gate"], w["up"], w["s_up"],
                                w["down"], w["s_down"])
    assert_close(out.cpu().numpy(), ref, "out")


def test_expert_ffn_fp8_skewed_and_limits():
    """Skewed routing at M = 16 (hot experts with up to 16 pairs in one
    column block, pairs past the first two loaded as they are reached), and
    the refusal beyond LDS: x of 16 tokens at H = 8192 is refused on the
    host, with nothing launched."""
    say("expert_ffn fp8 skewed, limits")
    M, H, I, E, k = 16, 1024, 512, 64, 8
    x = synth.activations(M, H, seed=5500)
    w = fp8_experts_host(H, I, E, 5501)
    idx, tw = synth.random_routing(M, E, k, 5502, 1.0)
    d = dev8(w)
    out = mv.moe_expert_ffn_fp8(to_dev(x), torch.from_numpy(idx).cuda(),
                                torch.from_numpy(tw).cuda(), d["gate"], d["s_gate"], d["up"],
                                d["s_up"], d["down"], d["s_down"])
    torch.cuda.synchronize()
    ref = oracle.expert_ffn_fp8(x, idx, tw, w["gate"], w["s_gate"], w["up"], w["s_up"],
                                w["down"], w["s_down"])
    assert_close(out.cpu().numpy(), ref, "out")
    H = 8192
    xb = torch.zeros((M, H), dtype=torch.bfloat16, device="cuda")
    qg = torch.zeros((E, I, H), dtype=torch.uint8, device="cuda")
    qd = torch.zeros((E, H, I), dtype=torch.uint8, device="cuda")
    sg = torch.ones((E, I), dtype=torch.float32, device="cuda")
    sd = torch.ones((E, H), dtype=torch.float32, device="cuda")
    with pytest.raises(mv.MoeError) as ei:
        mv.moe_expert_ffn_fp8(xb, torch.from_numpy(idx).cuda(), torch.from_numpy(tw).cuda(),
                              qg, sg, qg, sg, qd, sd)
    assert ei.value.status == 3


@pytest.fixture(scope="module")
def full_layer8():
    say("generating full-size fp8 layer weights on the device")
    H, E, I = 2560, 512, 1024
    K = synth.KIND
    qg, sg = synth.device_fp8_rows((E, I, H), synth.WEIGHT_STD, synth.WEIGHT_SEED, 0, K["gate"])
    qu, su = synth.device_fp8_rows((E, I, H), synth.WEIGHT_STD, synth.WEIGHT_SEED, 0, K["up"])
    qd, sd = synth.device_fp8_rows((E, H, I), synth.WEIGHT_STD, synth.WEIGHT_SEED, 0, K["down"])
    router = synth.device_normal_bf16((E, H), synth.WEIGHT_STD, synth.WEIGHT_SEED, 0, K["router"])
    return dict(router=router, gate=qg, s_gate=sg, up=qu, s_up=su, down=qd, s_down=sd)


@pytest.mark.parametrize("M,alpha", [(1, None), (6, None), (9, None), (10, None), (16, None),
                                     (16, 1.0)])
def test_layer_fp8_full_size(full_layer8, M, alpha):
    say("layer fp8 full size", M, alpha)
    k = 8
    L = full_layer8
    x = synth.activations(M, 2560, seed=5600 + M)
    bias = None if alpha is None else synth.zipf_bias(512, alpha)
    gi, gw, go = mv.moe_layer_fp8(to_dev(x), L["router"], L["gate"], L["s_gate"], L["up"],
                                  L["s_up"], L["down"], L["s_down"], k,
                                  None if bias is None else torch.from_numpy(bias).cuda())
    torch.cuda.synchronize()
    gi, gw, go = gi.cpu().numpy(), gw.cpu().numpy(), go.cpu().numpy()
    ref = oracle.route(x, to_host_bits(L["router"]), bias, k)
    same = compare_route(gi, gw, None, ref, k)
    assert len(same) >= M - 1, "more than one near-tie in a handful of tokens"

    def ffn8(xr, ids, w):
        # the oracle on the experts listed in ids, reading back just those
        uniq, inv = np.unique(ids, return_inverse=True)
        sel = torch.as_tensor(uniq, dtype=torch.long, device="cuda")
        sub = {key: L[key].index_select(0, sel).cpu().numpy()
               for key in ("gate", "s_gate", "up", "s_up", "down", "s_down")}
        return oracle.expert_ffn_fp8(xr, inv.reshape(ids.shape).astype(np.int32), w,
                                     sub["gate"], sub["s_gate"], sub["up"], sub["s_up"],
                                     sub["down"], sub["s_down"])

    out = ffn8(x, ref["idx"], ref["w"])
    assert_close(go[same], out[same], "out")
    check_tie_rows(x, gi, gw, go, ref, ffn8)
