"""Pins for the CPU oracle: facts that hold independently of the oracle's code.

Each ``pin_*`` takes an ``oracle.Oracle`` and raises AssertionError when the
oracle disagrees with something fixed outside it: a library routine (numpy
matmul, stable argsort, argmax, scipy's logistic function), a closed form on
planted inputs, or an invariant of the mathematics. The mutation test runs
every pin against copies of the oracle with planted mistakes to show that each
mistake is caught.

The method is the one in the LMSYS post "Chasing the batch-1 floor:
Ling-3.0-flash speculative decode on Blackwell".
"""
from __future__ import annotations

import math

import numpy as np
from scipy.special import expit

import synth

F = synth.bf16_to_f32


def _bits(values) -> np.ndarray:
    """bf16 bits of values that are exactly representable in bf16."""
    v = np.asarray(values, dtype=np.float32)
    b = synth.bf16_bits(v)
    assert np.array_equal(F(b), v), "planted value is not exact in bf16"
    return b


def _silu(z):
    return z * expit(z)


# --------------------------------------------------------------------- bf16

def pin_bf16_decode(o):
    """bf16 is the top half of binary32: a few patterns with known values."""
    cases = {0x3F80: 1.0, 0xBF80: -1.0, 0x4049: 3.140625, 0x0000: 0.0,
             0x0001: 2.0 ** -133, 0x0080: 2.0 ** -126,
             0x7F7F: (2.0 - 2.0 ** -7) * 2.0 ** 127, 0xC2F7: -123.5}
    for bits, val in cases.items():
        assert o.bf16_value(bits) == val, hex(bits)


# ------------------------------------------------------------------- router

def pin_route_logits_match_matmul(o):
    """Logits equal numpy's fp64 x @ Wg^T + bias on a non-square case."""
    M, H, E, k = 3, 40, 24, 5
    x = synth.normal_bf16((M, H), 1.0, 11, 1)
    wg = synth.normal_bf16((E, H), 0.02, 11, 2)
    bias = synth.rng(11, 3).normal(size=E).astype(np.float32) * 0.05
    r = o.route(x, wg, bias, k)
    ref = F(x).astype(np.float64) @ F(wg).astype(np.float64).T + bias.astype(np.float64)
    assert np.allclose(r["logits"], ref, rtol=0, atol=1e-12)


def pin_route_topk_matches_stable_argsort(o):
    """Selection equals numpy's stable argsort of the fp32 logits, with
    planted exact ties (duplicated router rows) resolved to the lower id."""
    M, H, E, k = 4, 32, 16, 4
    x = synth.normal_bf16((M, H), 1.0, 12, 1)
    wg = synth.normal_bf16((E, H), 0.02, 12, 2)
    wg[9] = wg[3]          # exact tie between experts 3 and 9
    wg[14] = wg[2]         # and between 2 and 14
    r = o.route(x, wg, None, k)
    with np.errstate(over="ignore"):
        l32 = r["logits"].astype(np.float32)
    for t in range(M):
        ref = np.argsort(-l32[t], kind="stable")[:k]
        assert np.array_equal(r["idx"][t], ref), (t, r["idx"][t], ref)
        sel = set(r["idx"][t].tolist())
        lo = min(l32[t, list(sel)])
        hi = max([l32[t, e] for e in range(E) if e not in sel])
        assert lo >= hi
    # planting the tie at the top: both copies of the largest row selected,
    # lower id first
    x1 = synth.normal_bf16((1, H), 1.0, 13, 1)
    wg1 = synth.normal_bf16((E, H), 0.02, 13, 2)
    top = int(np.argmax(F(x1)[0] @ F(wg1).T))
    wg1[0] = wg1[top]
    r1 = o.route(x1, wg1, None, 2)
    assert r1["idx"][0].tolist() == sorted([0, top])


def pin_route_planted_closed_form(o):
    """One-hot token against planted router rows: logits are the planted
    values and the weights are a softmax of them, in closed form."""
    H, E, k = 8, 6, 3
    vals = [0.5, -1.0, 2.0, 2.0, 0.0, -3.0]
    x = _bits([[1.0] + [0.0] * (H - 1)])
    wg = np.zeros((E, H), np.uint16)
    for e, v in enumerate(vals):
        wg[e, 0] = _bits([v])[0]
    r = o.route(x, wg, None, k)
    assert r["idx"][0].tolist() == [2, 3, 0]
    den = 2 * math.exp(2.0) + math.exp(0.5)
    exp_w = [math.exp(2.0) / den, math.exp(2.0) / den, math.exp(0.5) / den]
    assert np.allclose(r["w"][0], exp_w, rtol=1e-14, atol=0)
    assert r["gap_order"][0] == 0.0          # experts 2 and 3 tie exactly
    assert r["gap_sel"][0] == 0.5            # 3rd (0.5) minus 4th (0.0)


def pin_route_zero_input(o):
    """x = 0 and no bias: all logits are 0, ids 0..k-1, weights exactly 1/k."""
    M, H, E, k = 2, 16, 12, 4
    x = np.zeros((M, H), np.uint16)
    wg = synth.normal_bf16((E, H), 0.02, 14, 2)
    r = o.route(x, wg, None, k)
    assert np.all(r["logits"] == 0.0)
    assert np.array_equal(r["idx"], np.tile(np.arange(k, dtype=np.int32), (M, 1)))
    assert np.all(r["w"] == 1.0 / k)


def pin_route_bias_semantics(o):
    """A constant bias changes no selection or weight (softmax is shift
    invariant); a large bias on one expert puts it first."""
    M, H, E, k = 3, 24, 16, 4
    x = synth.normal_bf16((M, H), 1.0, 15, 1)
    wg = synth.normal_bf16((E, H), 0.02, 15, 2)
    r0 = o.route(x, wg, None, k)
    r1 = o.route(x, wg, np.full(E, 0.25, np.float32), k)
    assert np.array_equal(r0["idx"], r1["idx"])
    assert np.allclose(r0["w"], r1["w"], rtol=1e-12, atol=0)
    b = np.zeros(E, np.float32)
    b[7] = 50.0
    r2 = o.route(x, wg, b, k)
    assert np.all(r2["idx"][:, 0] == 7)
    assert np.all(r2["w"][:, 0] > 0.999)


def pin_route_weight_identities(o):
    """Weights sum to one, do not increase along the slots, and equal the
    full-softmax-then-renormalise route (the full denominator cancels)."""
    M, H, E, k = 5, 64, 32, 8
    x = synth.normal_bf16((M, H), 1.0, 16, 1)
    wg = synth.normal_bf16((E, H), 0.05, 16, 2)
    r = o.route(x, wg, synth.zipf_bias(E, 1.0), k)
    assert np.allclose(r["w"].sum(axis=1), 1.0, rtol=0, atol=1e-14)
    assert np.all(np.diff(r["w"], axis=1) <= 1e-15)
    assert np.allclose(r["w"], r["w_full"], rtol=1e-12, atol=0)
    # weights are the softmax of the selected logits: ratio of two weights
    # is exp of the logit difference
    for t in range(M):
        l = r["logits"][t, r["idx"][t]]
        assert np.allclose(r["w"][t] / r["w"][t, 0], np.exp(l - l[0]), rtol=1e-12)


def pin_route_gaps(o):
    """Near-tie gaps equal the differences of numpy's sorted logits."""
    M, H, E, k = 3, 32, 20, 6
    x = synth.normal_bf16((M, H), 1.0, 17, 1)
    wg = synth.normal_bf16((E, H), 0.02, 17, 2)
    r = o.route(x, wg, None, k)
    s = -np.sort(-r["logits"], axis=1)
    assert np.array_equal(r["gap_sel"], s[:, k - 1] - s[:, k])
    assert np.array_equal(r["gap_order"], np.min(s[:, :k - 1] - s[:, 1:k], axis=1))


# ------------------------------------------------------------------ experts

def pin_ffn_single_expert_is_dense_swiglu(o):
    """k = 1, weight 1: the layer is one dense SwiGLU MLP,
    Wd (silu(Wg x) * (Wu x)), here with numpy matmuls and scipy's logistic."""
    M, H, I, E = 3, 40, 24, 4
    x = synth.normal_bf16((M, H), 1.0, 21, 1)
    wgt = synth.layer_weights(H, E, I, seed=21)
    # N(0, 0.02) weights give |g| ~ 0.1; rescale so silu's curvature matters
    for key in ("gate", "up", "down"):
        wgt[key] = synth.bf16_bits(F(wgt[key]) * 8)
    idx = np.array([[2], [0], [3]], np.int32)
    w = np.ones((M, 1))
    out = o.expert_ffn(x, idx, w, wgt["gate"], wgt["up"], wgt["down"])
    xf = F(x).astype(np.float64)
    for t in range(M):
        e = idx[t, 0]
        g = F(wgt["gate"][e]).astype(np.float64) @ xf[t]
        u = F(wgt["up"][e]).astype(np.float64) @ xf[t]
        ref = F(wgt["down"][e]).astype(np.float64) @ (_silu(g) * u)
        assert np.allclose(out[t], ref, rtol=1e-11, atol=1e-13), t


def pin_ffn_silu_closed_forms(o):
    """Planted one-hot weights make g = (z, -z) and u = (1, 1), so the down
    rows read silu(z) - silu(-z) = z and silu(z) + silu(-z) = z tanh(z/2)."""
    H, I, E = 4, 2, 1
    for z in (0.0, 0.75, -2.5, 6.0, 0.015625):
        x = _bits([[z, 1.0, 0.0, 0.0]])
        wg = np.zeros((E, I, H), np.uint16)
        wu = np.zeros((E, I, H), np.uint16)
        wd = np.zeros((E, H, I), np.uint16)
        wg[0, 0, 0] = _bits([1.0])[0]
        wg[0, 1, 0] = _bits([-1.0])[0]
        wu[0, 0, 1] = wu[0, 1, 1] = _bits([1.0])[0]
        wd[0, 0] = _bits([1.0, -1.0])
        wd[0, 1] = _bits([1.0, 1.0])
        wd[0, 2] = _bits([1.0, 0.0])
        out, act = o.expert_ffn(x, np.zeros((1, 1), np.int32), np.ones((1, 1)),
                                wg, wu, wd, want_act=True)
        assert math.isclose(out[0, 0], z, rel_tol=1e-14, abs_tol=1e-15), z
        assert math.isclose(out[0, 1], z * math.tanh(z / 2), rel_tol=1e-13, abs_tol=1e-15), z
        assert math.isclose(out[0, 2], float(_silu(z)), rel_tol=1e-14, abs_tol=1e-15), z
        assert out[0, 3] == 0.0
        assert math.isclose(act[0, 0, 0], float(_silu(z)), rel_tol=1e-14, abs_tol=1e-15)
    # silu(0) is exactly 0
    x = _bits([[0.0, 1.0, 0.0, 0.0]])
    out = o.expert_ffn(x, np.zeros((1, 1), np.int32), np.ones((1, 1)), wg, wu, wd)
    assert np.all(out == 0.0)


def pin_ffn_dense_soft_moe(o):
    """k = E with the router's own weights: the layer is the dense soft MoE
    sum_e softmax_e(l) * SwiGLU_e(x), computed here with numpy."""
    M, H, I, E = 2, 32, 16, 6
    x = synth.normal_bf16((M, H), 1.0, 22, 1)
    wgt = synth.layer_weights(H, E, I, seed=22)
    for key in ("gate", "up", "down"):
        wgt[key] = synth.bf16_bits(F(wgt[key]) * 8)
    r = o.route(x, wgt["router"], None, E)
    out = o.expert_ffn(x, r["idx"], r["w"], wgt["gate"], wgt["up"], wgt["down"])
    xf = F(x).astype(np.float64)
    logits = xf @ F(wgt["router"]).astype(np.float64).T
    p = np.exp(logits - logits.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    for t in range(M):
        ref = np.zeros(H)
        for e in range(E):
            g = F(wgt["gate"][e]).astype(np.float64) @ xf[t]
            u = F(wgt["up"][e]).astype(np.float64) @ xf[t]
            ref += p[t, e] * (F(wgt["down"][e]).astype(np.float64) @ (_silu(g) * u))
        assert np.allclose(out[t], ref, rtol=1e-10, atol=1e-13)


def pin_ffn_linearity_and_relabeling(o):
    """Doubling W_down doubles the output exactly; the output is linear in the
    routing weights; relabeling experts (moving their slabs and ids together)
    leaves it bitwise unchanged."""
    M, H, I, E, k = 2, 24, 16, 6, 3
    x = synth.normal_bf16((M, H), 1.0, 23, 1)
    wgt = synth.layer_weights(H, E, I, seed=23)
    idx = np.array([[4, 1, 5], [1, 0, 2]], np.int32)
    w = np.array([[0.5, 0.3, 0.2], [0.6, 0.25, 0.15]])
    out = o.expert_ffn(x, idx, w, wgt["gate"], wgt["up"], wgt["down"])
    wd2 = synth.bf16_bits(F(wgt["down"]) * 2)
    out2 = o.expert_ffn(x, idx, w, wgt["gate"], wgt["up"], wd2)
    assert np.array_equal(out2, 2 * out)
    # linear in w: one-hot weights per slot sum back to the full result
    parts = []
    for j in range(k):
        wj = np.zeros_like(w)
        wj[:, j] = w[:, j]
        parts.append(o.expert_ffn(x, idx, wj, wgt["gate"], wgt["up"], wgt["down"]))
    assert np.allclose(sum(parts), out, rtol=1e-13, atol=1e-16)
    # slot j alone with weight 1 is that expert's own output; every slot
    # contributes (a dropped slot would leave its part at zero)
    for j in range(k):
        assert np.any(parts[j] != 0.0)
    perm = np.array([3, 5, 0, 4, 2, 1])        # new id of old expert e
    inv = np.argsort(perm)
    out_p = o.expert_ffn(x, perm[idx].astype(np.int32), w, wgt["gate"][inv],
                         wgt["up"][inv], wgt["down"][inv])
    assert np.array_equal(out_p, out)


def pin_ffn_rejects_bad_ids(o):
    x = np.zeros((1, 8), np.uint16)
    wg = np.zeros((2, 4, 8), np.uint16)
    wd = np.zeros((2, 8, 4), np.uint16)
    for bad in (-1, 2):
        try:
            o.expert_ffn(x, np.array([[bad]], np.int32), np.ones((1, 1)), wg, wg, wd)
        except ValueError:
            continue
        raise AssertionError("out-of-range expert id accepted")


# ------------------------------------------------------------------ lm_head

def pin_lmhead_matches_numpy_argmax(o):
    """Greedy token equals numpy's first-occurrence argmax of the fp32-rounded
    logits; zmax and gap match numpy's fp64 logits."""
    M, H, V = 3, 64, 300
    h = synth.normal_bf16((M, H), 1.0, 31, 1)
    wl = synth.normal_bf16((V, H), 0.02, 31, 2)
    wl[200] = wl[57]                         # duplicated rows: an exact tie
    r = o.lmhead(h, wl)
    z = F(h).astype(np.float64) @ F(wl).astype(np.float64).T
    tok = np.argmax(z.astype(np.float32), axis=1)
    assert np.array_equal(r["tok"], tok)
    assert np.array_equal(r["zmax"], z[np.arange(M), tok])
    s = -np.sort(-z, axis=1)
    assert np.array_equal(r["gap"], s[:, 0] - s[:, 1])


def pin_lmhead_planted(o):
    """A row equal to the hidden state wins (also at the first and last row);
    duplicated winners resolve to the lower id; a zero hidden state gives
    token 0."""
    M, H, V = 4, 32, 64
    h = synth.normal_bf16((M, H), 1.0, 32, 1)
    wl = synth.normal_bf16((V, H), 0.02, 32, 2)
    wl[41] = h[0]
    wl[13] = h[1]
    wl[50] = h[1]
    wl[V - 1] = h[2]
    wl[0] = h[3]
    r = o.lmhead(h, wl)
    assert r["tok"].tolist() == [41, 13, V - 1, 0]
    assert r["gap"][1] == 0.0
    r0 = o.lmhead(np.zeros((1, H), np.uint16), wl)
    assert r0["tok"].tolist() == [0]


# ---------------------------------------------------------------------- fp8

def pin_e4m3_decode(o):
    """Every E4M3 code against torch's float8_e4m3fn decode (NaN codes NaN),
    and hand values: 0x01 = 2^-9, 0x07 = 7 * 2^-9, 0x08 = 2^-6 (smallest
    normal), 0x38 = 1, 0x3C = 1.5, 0x7E = 448, 0xB8 = -1, 0x80 = -0."""
    import torch
    ref = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn)
    ref = ref.to(torch.float64).numpy()
    got = np.array([o.e4m3_value(q) for q in range(256)])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan) and nan.sum() == 2
    assert np.array_equal(got[~nan], ref[~nan])
    hand = {0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x38: 1.0, 0x3C: 1.5,
            0x7E: 448.0, 0xB8: -1.0}
    assert all(o.e4m3_value(q) == v for q, v in hand.items())
    z = o.e4m3_value(0x80)
    assert z == 0.0 and math.copysign(1.0, z) < 0


def _fp8_case(M, H, I, E, seed, pow2_scales):
    rng = np.random.default_rng(seed)
    def codes(shape):
        q = rng.integers(0, 256, size=shape).astype(np.uint8)
        q[(q & 0x7F) == 0x7F] = 0x3C                # no NaN codes
        return q
    def scales(shape):
        if pow2_scales:
            return np.ldexp(1.0, rng.integers(-12, -4, size=shape)).astype(np.float32)
        return rng.uniform(0.001, 0.01, size=shape).astype(np.float32)
    q = dict(gate=codes((E, I, H)), up=codes((E, I, H)), down=codes((E, H, I)))
    sc = dict(gate=scales((E, I)), up=scales((E, I)), down=scales((E, H)))
    return q, sc


def _dequant_bf16(o, q, s):
    """Exact bf16 bits of e4m3(q) * s for power-of-two scales."""
    table = np.array([o.e4m3_value(c) for c in range(256)])
    v = table[q] * s[..., None].astype(np.float64)
    return _bits(v.astype(np.float32))


def pin_expert_ffn_fp8_is_bf16_on_dequantised(o):
    """With power-of-two scales every dequantised weight is exact in bf16, so
    the fp8 FFN must equal the bf16 FFN on those values bit for bit; doubling
    every down scale doubles the output exactly; an expert's weights only
    matter through its own rows (a second expert's scales change nothing for
    tokens that do not use it)."""
    M, H, I, E, k = 3, 32, 16, 4, 2
    q, sc = _fp8_case(M, H, I, E, 61, True)
    x = synth.normal_bf16((M, H), 1.0, 61, 1)
    idx = np.array([[0, 2], [2, 1], [3, 0]], np.int32)
    w = np.array([[0.7, 0.3], [0.5, 0.5], [0.9, 0.1]])
    out8 = o.expert_ffn_fp8(x, idx, w, q["gate"], sc["gate"], q["up"], sc["up"],
                            q["down"], sc["down"])
    ref = o.expert_ffn(x, idx, w, _dequant_bf16(o, q["gate"], sc["gate"]),
                       _dequant_bf16(o, q["up"], sc["up"]), _dequant_bf16(o, q["down"], sc["down"]))
    assert np.array_equal(out8, ref)
    out2 = o.expert_ffn_fp8(x, idx, w, q["gate"], sc["gate"], q["up"], sc["up"],
                            q["down"], sc["down"] * 2)
    assert np.array_equal(out2, out8 * 2)
    sg = sc["gate"].copy()
    sg[1] *= 4                                    # expert 1: used by token 1 only
    out3 = o.expert_ffn_fp8(x, idx, w, q["gate"], sg, q["up"], sc["up"], q["down"], sc["down"])
    assert np.array_equal(out3[[0, 2]], out8[[0, 2]]) and not np.array_equal(out3[1], out8[1])


def pin_lmhead_fp8(o):
    """The fp8 lm_head equals the bf16 lm_head on the dequantised rows
    (power-of-two scales); a row whose scale is raised far enough wins."""
    M, H, V = 3, 32, 200
    rng = np.random.default_rng(62)
    q = rng.integers(0, 256, size=(V, H)).astype(np.uint8)
    q[(q & 0x7F) == 0x7F] = 0x38
    s = np.ldexp(1.0, rng.integers(-10, -6, size=V)).astype(np.float32)
    h = synth.normal_bf16((M, H), 1.0, 62, 1)
    r8 = o.lmhead_fp8(h, q, s)
    table = np.array([o.e4m3_value(c) for c in range(256)])
    wl = _bits((table[q] * s[:, None]).astype(np.float32))
    r16 = o.lmhead(h, wl)
    for key in ("tok", "zmax", "gap"):
        assert np.array_equal(r8[key], r16[key]), key
    z = (table[q] * s[:, None]) @ F(h).astype(np.float64).T        # [V, M]
    v_pos = int(np.argmax(z[:, 0]))                                 # make another row win token 0
    other = (v_pos + 7) % V
    if z[other, 0] > 0:
        s2 = s.copy()
        s2[other] = s[other] * 2.0 ** 12
        assert o.lmhead_fp8(h, q, s2)["tok"][0] == other


# ------------------------------------------------------------------ RMSNorm

def pin_rmsnorm_hand_examples(o):
    """Worked by hand. h = [3, 4], gain 1, eps 0: mean square 12.5, so the
    values are 3/sqrt(12.5) = 0.848528... = 1.697056 * 2^-1 (fraction
    0.697056 * 128 = 89.22 -> 89: bits 126 << 7 | 89 = 0x3F59) and
    4/sqrt(12.5) = 1.131371 (fraction 16.82 -> 17: 127 << 7 | 17 = 0x3F91).
    h = [0.5, 0.5], eps 1: mean square 0.25 + 1 = 1.25, 0.5/sqrt(1.25) =
    0.447214 = 1.788854 * 2^-2 (fraction 100.97 -> 101: 125 << 7 | 101 =
    0x3EE5). h = [1.5, 0, 0, 0], gain [1 + 3/128, 1, 1, 1], eps 0.4375: mean
    square 0.5625 + 0.4375 = 1 exactly, value 1.5 * 1.0234375 = 1.53515625,
    a tie between fractions 68 and 69 -> the even 68 (0x3FC4)."""
    one = 0x3F80
    xn = o.rmsnorm(_bits([[3.0, 4.0]]), np.array([one, one], np.uint16), 0.0)
    assert xn.tolist() == [[0x3F59, 0x3F91]]
    xn = o.rmsnorm(_bits([[0.5, 0.5]]), np.array([one, one], np.uint16), 1.0)
    assert xn.tolist() == [[0x3EE5, 0x3EE5]]
    xn = o.rmsnorm(_bits([[1.5, 0.0, 0.0, 0.0]]), _bits([1.0234375, 1.0, 1.0, 1.0]), 0.4375)
    assert xn.tolist() == [[0x3FC4, 0, 0, 0]]


def pin_rmsnorm_closed_forms(o):
    """eps = 0, gain 1: a constant row normalises to +-1 exactly; scaling a
    row by a power of two leaves the result bitwise unchanged; doubling the
    gain doubles every value exactly; the fp64 values have unit mean square;
    permuting the columns (with the gain) permutes the result."""
    H = 64
    rng = np.random.default_rng(11)
    one = np.full(H, 0x3F80, np.uint16)
    xn = o.rmsnorm(_bits([[-2.5] * H, [0.375] * H]), one, 0.0)
    assert np.all(xn[0] == 0xBF80) and np.all(xn[1] == 0x3F80)
    h = synth.normal_bf16((3, H), 1.0, 41, 1)
    g = synth.normal_bf16((H,), 1.0, 41, 2)
    base, ex = o.rmsnorm(h, g, 0.0, want_exact=True)
    assert np.array_equal(o.rmsnorm(_bits(F(h) * 8.0), g, 0.0), base)
    two = o.rmsnorm(h, _bits(F(g) * 2.0), 0.0)
    assert np.array_equal(F(two), F(base) * 2.0)
    _, ex1 = o.rmsnorm(h, one, 0.0, want_exact=True)
    assert np.allclose(np.mean(ex1 ** 2, axis=1), 1.0, rtol=0, atol=1e-14)
    perm = rng.permutation(H)
    assert np.array_equal(o.rmsnorm(h[:, perm], g[perm], 0.0), base[:, perm])


def pin_rmsnorm_rounds_to_nearest(o):
    """Every output is the bf16 value nearest to the fp64 value (neither
    neighbour is closer; an exact tie takes the even significand), on random
    rows with eps > 0."""
    h = synth.normal_bf16((4, 256), 3.0, 43, 1)
    g = synth.normal_bf16((256,), 1.0, 43, 2)
    xn, ex = o.rmsnorm(h, g, 1e-6, want_exact=True)
    b = xn.astype(np.int64)
    val = F(xn).astype(np.float64)
    up = F(((b + 1) & 0xFFFF).astype(np.uint16)).astype(np.float64)
    dn = F(((b - 1) & 0xFFFF).astype(np.uint16)).astype(np.float64)
    d = np.abs(ex - val)
    assert np.all(d <= np.abs(ex - up)) and np.all(d <= np.abs(ex - dn))
    tie = (d == np.abs(ex - up)) | (d == np.abs(ex - dn))
    assert np.all((b[tie] & 1) == 0)
    assert np.all(np.sign(val[ex != 0]) == np.sign(ex[ex != 0]))


# ----------------------------------------------------------- greedy verdict

def pin_verdict_planted_chains(o):
    """Chains built from the target's tokens: a chain that follows every
    prediction is accepted whole (M tokens committed, bonus tok[M-1]); a
    candidate changed at position j ends the prefix there (j tokens, bonus
    tok[j-1]) whatever follows it; the root never matters; a one-position
    chain commits just the bonus token."""
    rng = np.random.default_rng(5)
    for M in (1, 2, 6, 16):
        tok = rng.integers(0, 157184, size=M).astype(np.int32)
        chain = np.concatenate([[rng.integers(0, 157184)], tok[:-1]]).astype(np.int32)
        assert o.greedy_verdict(chain, tok) == (M, int(tok[M - 1]))
        for j in range(1, M):
            bad = chain.copy()
            bad[j] = tok[j - 1] + 1          # rejected; every later one still matches
            assert o.greedy_verdict(bad, tok) == (j, int(tok[j - 1]))
        root = chain.copy()
        root[0] = -7
        assert o.greedy_verdict(root, tok) == (M, int(tok[M - 1]))


def pin_verdict_brute_force(o):
    """Every chain over a two-token vocabulary at M = 5 against the target's
    tokens: the accept length is one plus the length of the run of pairwise
    equal (candidate, previous prediction) pairs from the start, and the
    committed tokens tok[0..n] are the accepted candidates followed by the
    bonus token."""
    import itertools
    M = 5
    for tok_bits in itertools.product((0, 1), repeat=M):
        tok = np.array(tok_bits, np.int32)
        for cand in itertools.product((0, 1), repeat=M - 1):
            chain = np.array((3,) + cand, np.int32)
            run = len(list(itertools.takewhile(lambda ab: ab[0] == ab[1],
                                               zip(chain[1:], tok[:-1]))))
            acc, bonus = o.greedy_verdict(chain, tok)
            assert acc == run + 1 and bonus == tok[run]
            committed = list(chain[1:acc]) + [bonus]
            assert committed == list(tok[:acc])


ALL_PINS = [v for k_, v in sorted(globals().items()) if k_.startswith("pin_")]
