"""Helpers for the GPU parity tests: uploads, readbacks, and the acceptance
rules (exact indices except at oracle-flagged near-ties, fp32 outputs within
max|err| <= 1e-2 * max|ref| per tensor)."""
from __future__ import annotations

import numpy as np
import torch

import oracle
import synth

#: fp32 acceptance: max |gpu - ref| <= REL_TOL * max |ref|, per tensor
REL_TOL = 1e-2
#: a top-k boundary or argmax whose fp64 gap is below this is a near-tie
TIE_BAND = 1e-3


def to_dev(bits: np.ndarray) -> torch.Tensor:
    """uint16 bf16 bits -> device bfloat16 tensor."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.to("cuda").view(torch.bfloat16)


def to_host_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def assert_close(gpu, ref, what: str, rel: float = REL_TOL):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape, (what, gpu.shape, ref.shape)
    scale = np.max(np.abs(ref)) if ref.size else 0.0
    err = np.max(np.abs(gpu - ref)) if ref.size else 0.0
    assert err <= rel * scale or (scale == 0.0 and err == 0.0), \
        f"{what}: max|err| {err:.3e} > {rel} * max|ref| {scale:.3e}"
    return err, scale


def check_selection(gidx: np.ndarray, logits64: np.ndarray, k: int):
    """A top-k row that differs from the oracle's must still be a valid top-k
    up to the near-tie band: distinct ids, descending logits within the band,
    and no unselected logit above the smallest selected one beyond the band."""
    assert len(set(gidx.tolist())) == k
    assert np.all((gidx >= 0) & (gidx < logits64.size))
    ls = logits64[gidx]
    assert np.all(ls[:-1] >= ls[1:] - TIE_BAND), ls
    rest = np.delete(logits64, gidx)
    if rest.size:
        assert rest.max() <= ls.min() + TIE_BAND


def compare_route(gidx, gw, glogits, ref, k):
    """Returns the rows whose selection equals the oracle's exactly."""
    M = gidx.shape[0]
    same = []
    for t in range(M):
        if np.array_equal(gidx[t], ref["idx"][t]):
            same.append(t)
            continue
        # any difference must sit at an oracle-flagged near-tie
        flagged = ref["gap_sel"][t] < TIE_BAND or ref["gap_order"][t] < TIE_BAND
        assert flagged, f"token {t}: ids {gidx[t]} != oracle {ref['idx'][t]} with no near-tie"
        check_selection(gidx[t], ref["logits"][t], k)
    if glogits is not None:
        assert_close(glogits, ref["logits"], "logits")
    if same:
        assert_close(gw[same], ref["w"][same], "topk_w")
        assert np.allclose(gw[same].sum(axis=1), 1.0, atol=1e-5)
    return same


def gather_experts(dev_w: dict, ids: np.ndarray):
    """Read back only the listed experts' slabs (bf16 bits) for the oracle."""
    sel = torch.as_tensor(ids, dtype=torch.long, device="cuda")
    return {key: to_host_bits(dev_w[key].index_select(0, sel)) for key in ("gate", "up", "down")}


def oracle_ffn_from_device(x_bits, idx, w, dev_w):
    """Oracle FFN on the experts listed in idx, reading back just those."""
    uniq, inv = np.unique(idx, return_inverse=True)
    sub = gather_experts(dev_w, uniq)
    return oracle.expert_ffn(x_bits, inv.reshape(idx.shape).astype(np.int32),
                             np.asarray(w, np.float64), sub["gate"], sub["up"], sub["down"])


def device_layer(H, E, I, layer=0, seed=synth.WEIGHT_SEED):
    """Full-size layer weights drawn on the device (torch generator)."""
    K = synth.KIND
    return dict(
        router=synth.device_normal_bf16((E, H), synth.WEIGHT_STD, seed, layer, K["router"]),
        gate=synth.device_normal_bf16((E, I, H), synth.WEIGHT_STD, seed, layer, K["gate"]),
        up=synth.device_normal_bf16((E, I, H), synth.WEIGHT_STD, seed, layer, K["up"]),
        down=synth.device_normal_bf16((E, H, I), synth.WEIGHT_STD, seed, layer, K["down"]),
    )


def check_tie_rows(x_bits, gi, gw, go, ref, ffn):
    """Rows where the GPU took another valid top-k at an oracle-flagged
    near-tie (compare_route already checked the set): the GPU's routing
    weights must be the softmax of the oracle's logits over the GPU's own
    set, and the GPU's output the oracle FFN on the GPU's own ids and
    weights. ffn(x_rows, idx, w) is the oracle FFN of the layer's experts.
    Returns the rows checked."""
    rows = [t for t in range(gi.shape[0]) if not np.array_equal(gi[t], ref["idx"][t])]
    if not rows:
        return rows
    for t in rows:
        lt = ref["logits"][t][gi[t]]
        wt = np.exp(lt - lt.max())
        assert_close(gw[t], wt / wt.sum(), f"topk_w of near-tie token {t}")
    out = ffn(x_bits[rows], gi[rows], gw[rows].astype(np.float64))
    assert_close(go[rows], out, "out of the near-tie tokens")
    return rows
