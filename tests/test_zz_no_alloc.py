"""moe_layer_noalloc through the C ABI: the same results as moe_layer with a
fresh workspace, on consecutive calls that share the library's per-GPU
scratch (a full-size layer, then smaller inputs that find the larger call's
data still in the array)."""
import ctypes

import numpy as np
import pytest
import torch

import moe_speculative_verify_amd as mv
import synth
from gpu_util import device_layer, to_dev

pytestmark = pytest.mark.gpu


def say(*a):
    print("CASE", *a, flush=True)


def layer_raw(L, fn, x, w, bias, M, H, I, E, k, ws=None):
    idx = torch.full((M, k), -7, dtype=torch.int32, device="cuda")
    tw = torch.full((M, k), -7.0, dtype=torch.float32, device="cuda")
    out = torch.full((M, H), -7.0, dtype=torch.float32, device="cuda")
    st = torch.cuda.current_stream().cuda_stream
    args = [x.data_ptr(), w["router"].data_ptr(), None if bias is None else bias.data_ptr(),
            w["gate"].data_ptr(), w["up"].data_ptr(), w["down"].data_ptr(), M, H, I, E, k,
            idx.data_ptr(), tw.data_ptr(), out.data_ptr()]
    if ws is not None:
        args += [ws.data_ptr(), ctypes.c_size_t(ws.numel())]
    rc = fn(*args, st)
    assert rc == 0, mv.status_str(rc)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), tw.cpu().numpy(), out.cpu().numpy()


def check_same(L, x, w, bias, M, H, I, E, k):
    ws = torch.zeros(L.moe_layer_workspace_bytes(M, H, I, E, k), dtype=torch.uint8,
                     device="cuda")
    ref = layer_raw(L, L.moe_layer, x, w, bias, M, H, I, E, k, ws)
    got = layer_raw(L, L.moe_layer_noalloc, x, w, bias, M, H, I, E, k)
    for a, b, what in zip(got, ref, ("topk_idx", "topk_w", "out")):
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), what


def test_noalloc_matches_moe_layer_on_consecutive_calls():
    assert torch.cuda.is_available()
    L = mv.lib()
    H, E, I, k = 2560, 512, 1024, 8
    w = device_layer(H, E, I, layer=3)
    bias = torch.from_numpy(synth.zipf_bias(E, 1.0)).cuda()
    # first call: the block-16 verify width (the MFMA down regime), Zipf routing
    say("noalloc full layer M=16 zipf")
    x16 = to_dev(synth.activations(16, H, seed=41))
    check_same(L, x16, w, bias, 16, H, I, E, k)
    # second call, smaller: one token, no bias (the GEMV regime)
    say("noalloc full layer M=1")
    x1 = to_dev(synth.activations(1, H, seed=42))
    check_same(L, x1, w, None, 1, H, I, E, k)
    del w
    # third call, smaller again: a ragged small layer
    M, H, E, I, k = 3, 264, 20, 136, 4
    say("noalloc small ragged", M, H, E, I, k)
    hw = synth.layer_weights(H, E, I, seed=synth.WEIGHT_SEED + 9)
    ws_ = {key: to_dev(hw[key]) for key in ("router", "gate", "up", "down")}
    xs = to_dev(synth.activations(M, H, seed=43))
    check_same(L, xs, ws_, None, M, H, I, E, k)


def test_noalloc_rejects_bad_shapes():
    L = mv.lib()
    A = 1 << 20
    # checked before the scratch is touched: nothing is launched
    assert L.moe_layer_noalloc(A, A, None, A, A, A, 17, 2560, 1024, 512, 8, A, A, A, None) == 3
    assert L.moe_layer_noalloc(None, A, None, A, A, A, 6, 2560, 1024, 512, 8, A, A, A, None) == 1
