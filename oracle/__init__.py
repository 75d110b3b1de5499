"""Plain fp64 CPU oracle for the batch-1 MoE verify hot path.

TEST INFRASTRUCTURE. Only the test suite, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package. It wraps
``oracle.c`` (plain C, double precision, ascending-index sums) through ctypes
and shares nothing with the GPU library.

The method is the one described in the LMSYS post "Chasing the batch-1 floor:
Ling-3.0-flash speculative decode on Blackwell": router gate matvec and top-k
(section "PDL: the latency floor of stacked small kernels", Fig. 7), expert
SwiGLU with an fp32 combine (section "Two fusions and a retune"), bf16 gate
and lm_head with a greedy verdict (section "bf16 router gate and lm_head").
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

_ERRORS = {-1: "null pointer", -2: "bad size", -3: "index out of range",
           -4: "non-finite input"}


def build(out: str = _LIB, src: str = _SRC) -> str:
    """Compile the oracle with gcc (-O2, no fast-math, OpenMP over outputs)."""
    tmp = out + ".tmp"
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC",
                           "-Wall", "-o", tmp, src, "-lm"])
    os.replace(tmp, out)
    return out


_P = ctypes.c_void_p
_I = ctypes.c_int32


class Oracle:
    """ctypes view of one compiled oracle library (the default, or a copy)."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        lib.oracle_bf16_value.argtypes = [ctypes.c_uint16]
        lib.oracle_bf16_value.restype = ctypes.c_double
        lib.oracle_route.argtypes = [_P, _P, _P, _I, _I, _I, _I,
                                     _P, _P, _P, _P, _P, _P]
        lib.oracle_route.restype = ctypes.c_int
        lib.oracle_expert_ffn.argtypes = [_P, _P, _P, _P, _P, _P,
                                          _I, _I, _I, _I, _I, _P, _P]
        lib.oracle_expert_ffn.restype = ctypes.c_int
        lib.oracle_lmhead.argtypes = [_P, _P, _I, _I, _I, _P, _P, _P]
        lib.oracle_lmhead.restype = ctypes.c_int
        lib.oracle_e4m3_value.argtypes = [ctypes.c_uint8]
        lib.oracle_e4m3_value.restype = ctypes.c_double
        lib.oracle_expert_ffn_fp8.argtypes = [_P] * 9 + [_I] * 5 + [_P]
        lib.oracle_expert_ffn_fp8.restype = ctypes.c_int
        lib.oracle_lmhead_fp8.argtypes = [_P, _P, _P, _I, _I, _I, _P, _P, _P]
        lib.oracle_lmhead_fp8.restype = ctypes.c_int
        lib.oracle_rmsnorm.argtypes = [_P, _P, ctypes.c_double, _I, _I, _P, _P]
        lib.oracle_rmsnorm.restype = ctypes.c_int
        lib.oracle_greedy_verdict.argtypes = [_P, _P, _I, _P]
        lib.oracle_greedy_verdict.restype = ctypes.c_int
        lib.oracle_set_threads.argtypes = [_I]
        lib.oracle_set_threads.restype = None
        lib.oracle_threads.argtypes = []
        lib.oracle_threads.restype = ctypes.c_int32
        self.lib = lib
        self.path = path

    def set_threads(self, n: int) -> int:
        """Use n OpenMP threads from now on; returns the count in effect."""
        self.lib.oracle_set_threads(int(n))
        return int(self.lib.oracle_threads())

    def threads(self) -> int:
        return int(self.lib.oracle_threads())

    @staticmethod
    def _check(rc: int, what: str) -> None:
        if rc != 0:
            raise ValueError(f"{what}: {_ERRORS.get(rc, rc)}")

    def bf16_value(self, bits: int) -> float:
        return self.lib.oracle_bf16_value(int(bits) & 0xFFFF)

    def route(self, x, wg, bias, k: int) -> dict:
        """x [M,H] u16, wg [E,H] u16, bias [E] f32 or None -> dict of arrays."""
        x = np.ascontiguousarray(x, dtype=np.uint16)
        wg = np.ascontiguousarray(wg, dtype=np.uint16)
        M, H = x.shape
        E, H2 = wg.shape
        if H2 != H:
            raise ValueError("router weight width does not match x")
        b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
        logits = np.empty((M, E), np.float64)
        idx = np.empty((M, k), np.int32)
        w = np.empty((M, k), np.float64)
        w_full = np.empty((M, k), np.float64)
        gap_sel = np.empty(M, np.float64)
        gap_order = np.empty(M, np.float64)
        rc = self.lib.oracle_route(
            x.ctypes.data, wg.ctypes.data, None if b is None else b.ctypes.data,
            M, H, E, k, logits.ctypes.data, idx.ctypes.data, w.ctypes.data,
            w_full.ctypes.data, gap_sel.ctypes.data, gap_order.ctypes.data)
        self._check(rc, "oracle_route")
        return dict(logits=logits, idx=idx, w=w, w_full=w_full,
                    gap_sel=gap_sel, gap_order=gap_order)

    def expert_ffn(self, x, idx, w, wgate, wup, wdown, want_act=False):
        """Selected experts' SwiGLU FFN + combine -> out [M,H] f64 (and act)."""
        x = np.ascontiguousarray(x, dtype=np.uint16)
        idx = np.ascontiguousarray(idx, dtype=np.int32)
        w = np.ascontiguousarray(w, dtype=np.float64)
        wgate = np.ascontiguousarray(wgate, dtype=np.uint16)
        wup = np.ascontiguousarray(wup, dtype=np.uint16)
        wdown = np.ascontiguousarray(wdown, dtype=np.uint16)
        M, H = x.shape
        _, k = idx.shape
        E, I, H2 = wgate.shape
        if H2 != H or wup.shape != wgate.shape or wdown.shape != (E, H, I):
            raise ValueError("expert weight shapes do not match")
        out = np.empty((M, H), np.float64)
        act = np.empty((M, k, I), np.float64) if want_act else None
        rc = self.lib.oracle_expert_ffn(
            x.ctypes.data, idx.ctypes.data, w.ctypes.data, wgate.ctypes.data,
            wup.ctypes.data, wdown.ctypes.data, M, H, I, E, k,
            out.ctypes.data, None if act is None else act.ctypes.data)
        self._check(rc, "oracle_expert_ffn")
        return (out, act) if want_act else out

    def lmhead(self, h, wlm) -> dict:
        """h [M,H] u16, wlm [V,H] u16 -> dict(tok, zmax, gap)."""
        h = np.ascontiguousarray(h, dtype=np.uint16)
        wlm = np.ascontiguousarray(wlm, dtype=np.uint16)
        M, H = h.shape
        V, H2 = wlm.shape
        if H2 != H:
            raise ValueError("lm_head width does not match h")
        tok = np.empty(M, np.int32)
        zmax = np.empty(M, np.float64)
        gap = np.empty(M, np.float64)
        rc = self.lib.oracle_lmhead(h.ctypes.data, wlm.ctypes.data, M, H, V,
                                    tok.ctypes.data, zmax.ctypes.data,
                                    gap.ctypes.data)
        self._check(rc, "oracle_lmhead")
        return dict(tok=tok, zmax=zmax, gap=gap)

    def e4m3_value(self, q: int) -> float:
        return self.lib.oracle_e4m3_value(int(q) & 0xFF)

    def expert_ffn_fp8(self, x, idx, w, qgate, sgate, qup, sup, qdown, sdown):
        """fp8 expert weights (E4M3 codes [E,I,H]/[E,H,I] u8, per-row fp32
        scales [E,I]/[E,H]) -> out [M,H] f64."""
        x = np.ascontiguousarray(x, dtype=np.uint16)
        idx = np.ascontiguousarray(idx, dtype=np.int32)
        w = np.ascontiguousarray(w, dtype=np.float64)
        qg, qu, qd = (np.ascontiguousarray(a, dtype=np.uint8) for a in (qgate, qup, qdown))
        sg, su, sd = (np.ascontiguousarray(a, dtype=np.float32) for a in (sgate, sup, sdown))
        M, H = x.shape
        _, k = idx.shape
        E, I, H2 = qg.shape
        if (H2 != H or qu.shape != qg.shape or qd.shape != (E, H, I) or sg.shape != (E, I)
                or su.shape != (E, I) or sd.shape != (E, H)):
            raise ValueError("fp8 expert shapes do not match")
        out = np.empty((M, H), np.float64)
        rc = self.lib.oracle_expert_ffn_fp8(
            x.ctypes.data, idx.ctypes.data, w.ctypes.data, qg.ctypes.data, sg.ctypes.data,
            qu.ctypes.data, su.ctypes.data, qd.ctypes.data, sd.ctypes.data, M, H, I, E, k,
            out.ctypes.data)
        self._check(rc, "oracle_expert_ffn_fp8")
        return out

    def lmhead_fp8(self, h, qlm, slm) -> dict:
        """h [M,H] u16, qlm [V,H] u8 E4M3, slm [V] f32 -> dict(tok, zmax, gap)."""
        h = np.ascontiguousarray(h, dtype=np.uint16)
        q = np.ascontiguousarray(qlm, dtype=np.uint8)
        sl = np.ascontiguousarray(slm, dtype=np.float32)
        M, H = h.shape
        V, H2 = q.shape
        if H2 != H or sl.shape != (V,):
            raise ValueError("fp8 lm_head shapes do not match")
        tok = np.empty(M, np.int32)
        zmax = np.empty(M, np.float64)
        gap = np.empty(M, np.float64)
        rc = self.lib.oracle_lmhead_fp8(h.ctypes.data, q.ctypes.data, sl.ctypes.data, M, H, V,
                                        tok.ctypes.data, zmax.ctypes.data, gap.ctypes.data)
        self._check(rc, "oracle_lmhead_fp8")
        return dict(tok=tok, zmax=zmax, gap=gap)

    def rmsnorm(self, h, gamma, eps: float, want_exact=False):
        """h [M,H] u16, gamma [H] u16 -> xn [M,H] u16 (bf16 bits) (, fp64 values)."""
        h = np.ascontiguousarray(h, dtype=np.uint16)
        gamma = np.ascontiguousarray(gamma, dtype=np.uint16)
        M, H = h.shape
        if gamma.shape != (H,):
            raise ValueError("gamma must be [H]")
        xn = np.empty((M, H), np.uint16)
        ex = np.empty((M, H), np.float64) if want_exact else None
        rc = self.lib.oracle_rmsnorm(h.ctypes.data, gamma.ctypes.data, float(eps), M, H,
                                     xn.ctypes.data, None if ex is None else ex.ctypes.data)
        self._check(rc, "oracle_rmsnorm")
        return (xn, ex) if want_exact else xn

    def greedy_verdict(self, tokens, tok) -> tuple[int, int]:
        """tokens [M] (root, drafted candidates), tok [M] (target argmax)
        -> (accept length n + 1, bonus token tok[n])."""
        tokens = np.ascontiguousarray(tokens, dtype=np.int32)
        tok = np.ascontiguousarray(tok, dtype=np.int32)
        if tokens.shape != tok.shape or tokens.ndim != 1:
            raise ValueError("tokens and tok must be two [M] vectors")
        acc = np.empty(2, np.int32)
        rc = self.lib.oracle_greedy_verdict(tokens.ctypes.data, tok.ctypes.data,
                                            tokens.shape[0], acc.ctypes.data)
        self._check(rc, "oracle_greedy_verdict")
        return int(acc[0]), int(acc[1])


_default: Oracle | None = None


def load() -> Oracle:
    """The default oracle library, compiled on first use if it is missing."""
    global _default
    if _default is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        _default = Oracle(_LIB)
    return _default


def set_threads(n):
    return load().set_threads(n)


def threads():
    return load().threads()


def route(x, wg, bias, k):
    return load().route(x, wg, bias, k)


def expert_ffn(x, idx, w, wgate, wup, wdown, want_act=False):
    return load().expert_ffn(x, idx, w, wgate, wup, wdown, want_act)


def lmhead(h, wlm):
    return load().lmhead(h, wlm)


def greedy_verdict(tokens, tok):
    return load().greedy_verdict(tokens, tok)


def rmsnorm(h, gamma, eps, want_exact=False):
    return load().rmsnorm(h, gamma, eps, want_exact)


def expert_ffn_fp8(x, idx, w, qgate, sgate, qup, sup, qdown, sdown):
    return load().expert_ffn_fp8(x, idx, w, qgate, sgate, qup, sup, qdown, sdown)


def lmhead_fp8(h, qlm, slm):
    return load().lmhead_fp8(h, qlm, slm)
