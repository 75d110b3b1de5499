"""Workload sizes against the figures the post prints (tests/golden)."""
import os

import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "model_facts.txt")


def _facts():
    out = {}
    for line in open(GOLDEN):
        if line.strip() and not line.startswith("#"):
            name, value, _ = line.split(" ", 2)
            out[name] = float(value)
    return out


def test_router_gate_is_2_6_mb_in_bf16():
    f = _facts()
    w = synth.WORKLOADS["gate"]
    assert w["E"] == f["experts"] and w["H"] == f["hidden"]
    nbytes = w["E"] * w["H"] * 2
    assert nbytes == 2_621_440
    assert round(nbytes / 1e6, 1) == f["gate_mb_bf16"]
    # fp32 would be twice that: bf16 "halves those bytes"
    assert (w["E"] * w["H"] * 4) / nbytes == f["gate_dtype_halving"]


def test_lm_head_shape():
    f = _facts()
    w = synth.WORKLOADS["lmhead"]
    assert w["H"] == f["hidden"] and w["M"] == f["verify_tokens_nextn"]
    assert abs(w["V"] - f["vocab_approx"]) / f["vocab_approx"] < 0.01
    assert w["V"] * w["H"] * 2 == 804_782_080


def test_layer_shapes():
    f = _facts()
    for name in ("layer_m1", "layer_m6", "layer_m16"):
        w = synth.WORKLOADS[name]
        assert w["E"] == f["experts"] and w["H"] == f["hidden"]
    assert synth.WORKLOADS["layer_m6"]["M"] == f["verify_tokens_nextn"]
    # per expert: gate + up + down rows, bf16
    per_expert = 3 * 1024 * 2560 * 2
    assert per_expert == 15_728_640
    # the post's ~94 MB per layer-step is below top-8 of one token at I=1024
    # (125.8 MB); I = 1024 is the fixed reading, the discrepancy is recorded
    assert 8 * per_expert > f["expert_mb_per_layer_step"] * 1e6
