"""GPU parity of the shared-expert variants (moe_expert_ffn_shared,
moe_layer_shared) against the fp64 CPU oracle.

The shared expert is one more SwiGLU expert that every token uses with
weight 1, summed after the routed slots: the oracle's own definition covers
it as a (k+1)-th slot whose expert is appended to the weight tensors. Rules
as everywhere: indices exact except at flagged near-ties, fp32 outputs within
1e-2 * max|ref| per tensor.
"""
import numpy as np
import pytest
import torch

import moe_speculative_verify_amd as mv
import oracle
import synth
from gpu_util import (assert_close, check_tie_rows, compare_route, device_layer, gather_experts,
                      to_dev, to_host_bits)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    mv.lib()
    yield
    torch.cuda.synchronize()


def say(*a):
    print("CASE", *a, flush=True)


def shared_weights_host(H, I, seed):
    return dict(gate=synth.normal_bf16((I, H), synth.WEIGHT_STD, seed, 71),
                up=synth.normal_bf16((I, H), synth.WEIGHT_STD, seed, 72),
                down=synth.normal_bf16((H, I), synth.WEIGHT_STD, seed, 73))


def oracle_with_shared(x, idx, w, routed, shared):
    """The oracle's expert FFN with the shared expert as slot k (id E)."""
    M, k = idx.shape
    E = routed["gate"].shape[0]
    idx2 = np.concatenate([idx, np.full((M, 1), E, np.int32)], axis=1)
    w2 = np.concatenate([np.asarray(w, np.float64), np.ones((M, 1))], axis=1)
    return oracle.expert_ffn(x, idx2, w2,
                             np.concatenate([routed["gate"], shared["gate"][None]]),
                             np.concatenate([routed["up"], shared["up"][None]]),
                             np.concatenate([routed["down"], shared["down"][None]]))


SHARED_CASES = [
    # M, H, I, E, k  (the last two rows run the MFMA down kernel: M*(k+1)*I*2 beyond LDS)
    (1, 256, 128, 16, 2),
    (6, 264, 136, 20, 4),
    (16, 256, 128, 16, 8),
    (3, 8, 8, 3, 2),
    (16, 256, 1032, 16, 8),
    (10, 512, 1024, 64, 8),
]


@pytest.mark.parametrize("M,H,I,E,k", SHARED_CASES)
def test_expert_ffn_shared_matches_oracle(M, H, I, E, k):
    say("expert_ffn_shared", M, H, I, E, k)
    x = synth.activations(M, H, seed=4000 + I)
    w = synth.layer_weights(H, E, I, seed=synth.WEIGHT_SEED + 40 + I)
    sw = shared_weights_host(H, I, 4100 + I)
    idx, tw = synth.random_routing(M, E, k, 4200 + M, 0.0)
    out = mv.moe_expert_ffn_shared(to_dev(x), torch.from_numpy(idx).cuda(),
                                   torch.from_numpy(tw).cuda(), to_dev(w["gate"]),
                                   to_dev(w["up"]), to_dev(w["down"]), to_dev(sw["gate"]),
                                   to_dev(sw["up"]), to_dev(sw["down"]))
    torch.cuda.synchronize()
    ref = oracle_with_shared(x, idx, tw, w, sw)
    assert_close(out.cpu().numpy(), ref, "out")


def test_shared_only_is_dense_swiglu_difference():
    """With and without the shared expert, on the same routing: the
    difference is the shared expert alone (within tolerance), and the call
    without it is unchanged bit for bit by the shared-expert code."""
    say("shared expert difference")
    M, H, I, E, k = 6, 256, 128, 16, 2
    x = synth.activations(M, H, seed=4301)
    w = synth.layer_weights(H, E, I, seed=synth.WEIGHT_SEED + 43)
    sw = shared_weights_host(H, I, 4302)
    idx, tw = synth.random_routing(M, E, k, 4303, 0.0)
    args = (to_dev(x), torch.from_numpy(idx).cuda(), torch.from_numpy(tw).cuda(),
            to_dev(w["gate"]), to_dev(w["up"]), to_dev(w["down"]))
    with_s = mv.moe_expert_ffn_shared(*args, to_dev(sw["gate"]), to_dev(sw["up"]),
                                      to_dev(sw["down"])).cpu().numpy()
    without = mv.moe_expert_ffn(*args).cpu().numpy()
    without2 = mv.moe_expert_ffn(*args).cpu().numpy()
    assert np.array_equal(without, without2)
    dense = oracle.expert_ffn(x, np.zeros((M, 1), np.int32), np.ones((M, 1)),
                              sw["gate"][None], sw["up"][None], sw["down"][None])
    assert_close(with_s - without, dense, "shared contribution")


@pytest.fixture(scope="module")
def full_layer():
    say("generating full-size layer weights on the device")
    L = device_layer(2560, 512, 1024)
    K = synth.KIND
    L["shared"] = dict(
        gate=synth.device_normal_bf16((1024, 2560), synth.WEIGHT_STD, synth.WEIGHT_SEED, 0, 50 + K["gate"]),
        up=synth.device_normal_bf16((1024, 2560), synth.WEIGHT_STD, synth.WEIGHT_SEED, 0, 50 + K["up"]),
        down=synth.device_normal_bf16((2560, 1024), synth.WEIGHT_STD, synth.WEIGHT_SEED, 0, 50 + K["down"]))
    return L


@pytest.mark.parametrize("M,alpha", [(1, None), (6, None), (16, 1.0)])
def test_layer_shared_full_size(full_layer, M, alpha):
    say("layer_shared full size", M, alpha)
    k = 8
    x = synth.activations(M, 2560, seed=4400 + M)
    bias = None if alpha is None else synth.zipf_bias(512, alpha)
    b = None if bias is None else torch.from_numpy(bias).cuda()
    S = full_layer["shared"]
    gi, gw, go = mv.moe_layer_shared(to_dev(x), full_layer["router"], full_layer["gate"],
                                     full_layer["up"], full_layer["down"], S["gate"], S["up"],
                                     S["down"], k, b)
    torch.cuda.synchronize()
    gi, gw, go = gi.cpu().numpy(), gw.cpu().numpy(), go.cpu().numpy()
    # the routing is moe_layer's, bit for bit
    pi, pw, _ = mv.moe_layer(to_dev(x), full_layer["router"], full_layer["gate"],
                             full_layer["up"], full_layer["down"], k, b)
    torch.cuda.synchronize()
    assert np.array_equal(pi.cpu().numpy(), gi) and np.array_equal(pw.cpu().numpy(), gw)
    ref = oracle.route(x, to_host_bits(full_layer["router"]), bias, k)
    same = compare_route(gi, gw, None, ref, k)
    assert len(same) >= M - 1, "more than one near-tie in a handful of tokens"
    sw = {key: to_host_bits(S[key]) for key in ("gate", "up", "down")}

    def ffn_shared(xr, ids, w):
        uniq, inv = np.unique(ids, return_inverse=True)
        sub = gather_experts(full_layer, uniq)
        return oracle_with_shared(xr, inv.reshape(ids.shape).astype(np.int32), w, sub, sw)

    out = ffn_shared(x, ref["idx"], ref["w"])
    assert_close(go[same], out[same], "out")
    check_tie_rows(x, gi, gw, go, ref, ffn_shared)
