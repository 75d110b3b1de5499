"""Seeded synthetic inputs for the batch-1 MoE verify hot path.

This module only draws random numbers and lays them out: it holds none of the
method's arithmetic (no dot product, softmax, top-k, activation or combine).
The tests, the bench and the smoke check take their inputs from here, and the
same arrays feed both the GPU library and the CPU oracle.

Shapes follow the model the LMSYS post "Chasing the batch-1 floor:
Ling-3.0-flash speculative decode on Blackwell" runs: 512 routed experts
(Fig. 2), a 2.6 MB bf16 router gate per MoE layer (section "Fix the ruler
before the machine"), hidden width 2560 and a vocabulary of about 157k
(the Indonesian summary page), verify widths of 1, 6 (NEXTN, draft_tokens=6)
and 16 (DSpark block) tokens. Weights are N(0, 0.02) and activations N(0, 1),
rounded to bf16.
"""
from __future__ import annotations

import numpy as np

#: seeds used everywhere (recorded with every bench line)
WEIGHT_SEED = 20260821
ACT_SEED = 1
ZIPF_SEED = 2

#: tensor kinds, part of a weight stream's identity
KIND = {"router": 0, "gate": 1, "up": 2, "down": 3, "lm_head": 4, "bias": 5}

#: the workloads, by name
WORKLOADS = {
    # one MoE layer small enough for a pure-loop oracle in well under a second
    "tiny": dict(H=256, E=16, I=128, k=2, M=1, V=None),
    # router gate only, 512 x 2560 bf16, six verify tokens
    "gate": dict(H=2560, E=512, I=None, k=8, M=6, V=None),
    # full MoE layer verify step
    "layer_m6": dict(H=2560, E=512, I=1024, k=8, M=6, V=None),
    "layer_m1": dict(H=2560, E=512, I=1024, k=8, M=1, V=None),
    "layer_m16": dict(H=2560, E=512, I=1024, k=8, M=16, V=None),
    # lm_head greedy step
    "lmhead": dict(H=2560, E=None, I=None, k=None, M=6, V=157184),
}

WEIGHT_STD = 0.02
ACT_STD = 1.0
ZIPF_S = 1.1


def bf16_bits(a) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest, ties to even."""
    f = np.ascontiguousarray(a, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_to_f32(bits) -> np.ndarray:
    """bf16 bit patterns -> float32 values (exact)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def rng(seed: int, *ids: int) -> np.random.Generator:
    """Independent PCG64 stream for (seed, ids...)."""
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, *ids])))


def normal_bf16(shape, std: float, seed: int, *ids: int) -> np.ndarray:
    """N(0, std^2) samples rounded to bf16, as uint16 bits."""
    g = rng(seed, *ids)
    v = g.standard_normal(size=shape, dtype=np.float32) * np.float32(std)
    return bf16_bits(v)


def activations(M: int, H: int, seed: int = ACT_SEED, tag: int = 0) -> np.ndarray:
    """Verify-token activations [M,H], N(0,1) in bf16."""
    return normal_bf16((M, H), ACT_STD, seed, 1000 + tag, M, H)


def hidden_states(M: int, H: int, seed: int = ACT_SEED, tag: int = 0,
                  std: float = 3.0) -> np.ndarray:
    """Hidden states before the router chain's norm [M,H]: N(0, std^2) in
    bf16 (a residual stream whose scale the norm removes)."""
    return normal_bf16((M, H), std, seed, 2000 + tag, M, H)


def norm_gain(H: int, seed: int = WEIGHT_SEED, layer: int = 0) -> np.ndarray:
    """Per-column gain of the norm [H]: 1 + N(0, 0.1^2), in bf16."""
    g = rng(seed, layer, 97, H)
    v = np.float32(1.0) + g.standard_normal(size=H, dtype=np.float32) * np.float32(0.1)
    return bf16_bits(v)


def fp8_rows(shape, std: float, seed: int, *ids: int):
    """fp8 weights of N(0, std^2) rows: (E4M3 codes uint8 [..., K], fp32
    scale per row [...]). Each row is scaled by its largest magnitude / 448
    and converted with torch's own float8_e4m3fn conversion (nearest, no
    saturation needed: every scaled value is within +-448)."""
    import torch

    g = rng(seed, *ids)
    v = g.standard_normal(size=shape, dtype=np.float32) * np.float32(std)
    amax = np.max(np.abs(v), axis=-1)
    scale = (np.where(amax > 0, amax, 1.0) / 448.0).astype(np.float32)
    t = torch.from_numpy(v / scale[..., None])
    codes = t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return codes, scale


def device_fp8_rows(shape, std: float, seed: int, *ids: int, device="cuda",
                    chunk_rows: int = 1 << 16):
    """fp8_rows drawn on the device (full-size tensors): (uint8 codes, fp32
    scales) torch tensors; values are deterministic for (seed, ids, shape)."""
    import torch

    K = shape[-1]
    rows = int(np.prod(shape[:-1]))
    codes = torch.empty((rows, K), dtype=torch.uint8, device=device)
    scales = torch.empty(rows, dtype=torch.float32, device=device)
    gen = torch.Generator(device=device)
    gen.manual_seed(int(np.random.SeedSequence([seed, *ids, 8]).generate_state(1)[0]))
    for r0 in range(0, rows, chunk_rows):
        r1 = min(rows, r0 + chunk_rows)
        v = torch.randn((r1 - r0, K), generator=gen, device=device, dtype=torch.float32) * std
        amax = v.abs().amax(dim=1)
        sc = torch.where(amax > 0, amax, torch.ones_like(amax)) / 448.0
        codes[r0:r1] = (v / sc[:, None]).to(torch.float8_e4m3fn).view(torch.uint8)
        scales[r0:r1] = sc
    return codes.view(*shape), scales.view(*shape[:-1])


def zipf_bias(E: int, alpha: float, seed: int = ZIPF_SEED, s: float = ZIPF_S) -> np.ndarray:
    """Router bias whose exponential follows a Zipf(s) popularity.

    Expert e gets popularity rank r_e = 1 + pi(e) for a seeded permutation pi
    (so popularity is uncorrelated with the expert id) and bias
    alpha * (-s * ln r_e), shifted to zero mean. alpha = 0 gives no skew.
    """
    perm = rng(seed, 77, E).permutation(E)
    r = 1.0 + perm.astype(np.float64)
    b = alpha * (-s * np.log(r))
    b -= b.mean()
    return b.astype(np.float32)


def random_routing(M: int, E: int, k: int, seed: int, skew: float = 0.0):
    """A routing decision drawn directly (for expert-FFN-only cases).

    Each token gets k distinct expert ids (drawn with probability proportional
    to exp(skew * zipf_bias)) and k positive weights that sum to one.
    """
    g = rng(seed, 31, M, E, k)
    p = np.exp(zipf_bias(E, skew).astype(np.float64)) if skew else np.ones(E)
    p /= p.sum()
    idx = np.stack([g.choice(E, size=k, replace=False, p=p) for _ in range(M)]).astype(np.int32)
    w = g.uniform(0.1, 1.0, size=(M, k))
    w = (w / w.sum(axis=1, keepdims=True)).astype(np.float32)
    return idx, w


def layer_weights(H: int, E: int, I: int, seed: int = WEIGHT_SEED, layer: int = 0):
    """Host-generated weights of one MoE layer (small shapes only)."""
    return dict(
        router=normal_bf16((E, H), WEIGHT_STD, seed, layer, KIND["router"]),
        gate=normal_bf16((E, I, H), WEIGHT_STD, seed, layer, KIND["gate"]),
        up=normal_bf16((E, I, H), WEIGHT_STD, seed, layer, KIND["up"]),
        down=normal_bf16((E, H, I), WEIGHT_STD, seed, layer, KIND["down"]),
    )


def device_normal_bf16(shape, std: float, seed: int, *ids: int, device="cuda",
                       chunk_elems: int = 1 << 27, out=None):
    """N(0, std^2) bf16 tensor drawn on the device with torch's generator.

    Used for the full-size weights (gigabytes), which are too slow to draw on
    the host. Values are deterministic for a given (seed, ids, shape, chunk).
    """
    import torch

    n = int(np.prod(shape))
    if out is None:
        out = torch.empty(n, dtype=torch.bfloat16, device=device)
    flat = out.view(-1)
    assert flat.numel() == n
    s = int(np.random.SeedSequence([seed, *ids]).generate_state(1, np.uint64)[0] >> 1)
    g = torch.Generator(device=device)
    g.manual_seed(s)
    for lo in range(0, n, chunk_elems):
        hi = min(n, lo + chunk_elems)
        tmp = torch.randn(hi - lo, generator=g, device=device, dtype=torch.float32)
        tmp.mul_(std)
        flat[lo:hi].copy_(tmp)
        del tmp
    return out.view(*shape)
