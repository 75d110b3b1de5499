"""Python binding of libmoeverify.so, the gfx950 MoE verify hot path.

Argument marshalling only: every step runs in the library's HIP kernels.
PyTorch supplies device memory and the current stream; nothing here computes.
The names match the C entry points declared in include/moe_verify.h.

bf16 tensors may be torch.bfloat16, torch.int16 or torch.uint16 (raw bits).
If the library is not built, importing works but every call raises
RuntimeError: there is no CPU fallback.
"""
from __future__ import annotations

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoeverify.so")

MOE_OK = 0
STATUS = {0: "MOE_OK", 1: "MOE_ERR_NULL", 2: "MOE_ERR_SHAPE", 3: "MOE_ERR_UNSUPPORTED",
          4: "MOE_ERR_ALIGN", 5: "MOE_ERR_WORKSPACE", 6: "MOE_ERR_LAUNCH"}

#: every symbol the header declares
EXPORTS = ("moe_abi_version", "moe_status_str", "moe_workspace_clear", "moe_hbm_read_probe",
           "moe_route_workspace_bytes", "moe_route", "moe_route_rmsnorm",
           "moe_expert_ffn_workspace_bytes", "moe_expert_ffn", "moe_expert_ffn_shared",
           "moe_expert_ffn_fp8", "moe_layer_fp8",
           "moe_layer_workspace_bytes", "moe_layer", "moe_layer_noalloc", "moe_layer_rmsnorm",
           "moe_layer_shared",
           "lmhead_argmax_workspace_bytes", "lmhead_argmax", "lmhead_greedy_verify",
           "lmhead_argmax_fp8", "lmhead_greedy_verify_fp8",
           "lmhead_partial_keys", "lmhead_partial_keys_fp8", "lmhead_merge_keys")


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn}: {STATUS.get(status, status)} ({status_str(status)})")
        self.status = status


_lib = None

_P = ctypes.c_void_p
_I = ctypes.c_int32
_S = ctypes.c_size_t


def lib() -> ctypes.CDLL:
    """The loaded library (RuntimeError if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"HIP library not built: {LIB_PATH} is missing "
                               "(run __graft_entry__.build())")
        L = ctypes.CDLL(LIB_PATH)
        L.moe_abi_version.restype = ctypes.c_int32
        L.moe_abi_version.argtypes = []
        L.moe_status_str.restype = ctypes.c_char_p
        L.moe_status_str.argtypes = [ctypes.c_int32]
        L.moe_workspace_clear.restype = ctypes.c_int32
        L.moe_workspace_clear.argtypes = [_P, _S, _P]
        L.moe_hbm_read_probe.restype = ctypes.c_int32
        L.moe_hbm_read_probe.argtypes = [_P, _S, _P, _P]
        L.moe_route_workspace_bytes.restype = _S
        L.moe_route_workspace_bytes.argtypes = [_I, _I]
        L.moe_route.restype = ctypes.c_int32
        L.moe_route.argtypes = [_P, _P, _P, _I, _I, _I, _I, _P, _P, _P, _P, _S, _P]
        L.moe_route_rmsnorm.restype = ctypes.c_int32
        L.moe_route_rmsnorm.argtypes = [_P, _P, ctypes.c_float, _P, _P, _I, _I, _I, _I,
                                        _P, _P, _P, _P, _P, _S, _P]
        L.moe_layer_rmsnorm.restype = ctypes.c_int32
        L.moe_layer_rmsnorm.argtypes = [_P, _P, ctypes.c_float, _P, _P, _P, _P, _P,
                                        _I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _S, _P]
        L.moe_expert_ffn_shared.restype = ctypes.c_int32
        L.moe_expert_ffn_shared.argtypes = [_P] * 9 + [_I] * 5 + [_P, _P, _S, _P]
        L.moe_expert_ffn_fp8.restype = ctypes.c_int32
        L.moe_expert_ffn_fp8.argtypes = [_P] * 9 + [_I] * 5 + [_P, _P, _S, _P]
        L.moe_layer_fp8.restype = ctypes.c_int32
        L.moe_layer_fp8.argtypes = [_P] * 9 + [_I] * 5 + [_P, _P, _P, _P, _S, _P]
        L.moe_layer_shared.restype = ctypes.c_int32
        L.moe_layer_shared.argtypes = [_P] * 9 + [_I] * 5 + [_P, _P, _P, _P, _S, _P]
        L.moe_expert_ffn_workspace_bytes.restype = _S
        L.moe_expert_ffn_workspace_bytes.argtypes = [_I, _I, _I, _I, _I]
        L.moe_expert_ffn.restype = ctypes.c_int32
        L.moe_expert_ffn.argtypes = [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I,
                                     _P, _P, _S, _P]
        L.moe_layer_noalloc.restype = ctypes.c_int32
        L.moe_layer_noalloc.argtypes = [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I,
                                        _P, _P, _P, _P]
        L.moe_layer_workspace_bytes.restype = _S
        L.moe_layer_workspace_bytes.argtypes = [_I, _I, _I, _I, _I]
        L.moe_layer.restype = ctypes.c_int32
        L.moe_layer.argtypes = [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I,
                                _P, _P, _P, _P, _S, _P]
        L.lmhead_argmax_workspace_bytes.restype = _S
        L.lmhead_argmax_workspace_bytes.argtypes = [_I, _I]
        L.lmhead_argmax.restype = ctypes.c_int32
        L.lmhead_argmax.argtypes = [_P, _P, _I, _I, _I, _P, _P, _P, _S, _P]
        L.lmhead_argmax_fp8.restype = ctypes.c_int32
        L.lmhead_argmax_fp8.argtypes = [_P, _P, _P, _I, _I, _I, _P, _P, _P, _S, _P]
        L.lmhead_greedy_verify_fp8.restype = ctypes.c_int32
        L.lmhead_greedy_verify_fp8.argtypes = [_P, _P, _P, _P, _I, _I, _I, _P, _P, _P, _P, _S, _P]
        L.lmhead_partial_keys.restype = ctypes.c_int32
        L.lmhead_partial_keys.argtypes = [_P, _P, _I, _I, _I, _P, _S, _P]
        L.lmhead_partial_keys_fp8.restype = ctypes.c_int32
        L.lmhead_partial_keys_fp8.argtypes = [_P, _P, _P, _I, _I, _I, _P, _S, _P]
        L.lmhead_merge_keys.restype = ctypes.c_int32
        L.lmhead_merge_keys.argtypes = [_I, _I, _P, _P, _P, _P, _P, _S, _P]
        L.lmhead_greedy_verify.restype = ctypes.c_int32
        L.lmhead_greedy_verify.argtypes = [_P, _P, _P, _I, _I, _I, _P, _P, _P, _P, _S, _P]
        _lib = L
    return _lib


def moe_abi_version() -> int:
    return lib().moe_abi_version()


def status_str(status: int) -> str:
    return lib().moe_status_str(int(status)).decode()


moe_status_str = status_str


def _check(fn: str, status: int) -> None:
    if status != MOE_OK:
        raise MoeError(fn, status)


# ----------------------------------------------------------- marshalling

_BF16 = (torch.bfloat16, torch.int16, torch.uint16)


def _ptr(t: torch.Tensor | None, name: str, dtypes=None, shape=None) -> int | None:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtypes is not None and t.dtype not in dtypes:
        raise ValueError(f"{name}: dtype {t.dtype} not in {dtypes}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)} != {tuple(shape)}")
    return t.data_ptr()


def _stream_obj(stream):
    return torch.cuda.current_stream() if stream is None else stream


def _stream(stream) -> int:
    return _stream_obj(stream).cuda_stream


class Workspace:
    """A zero-filled device workspace, grown on demand, one per (kind,
    device, stream).

    The library leaves every counter it uses at zero, so a workspace is
    reused across calls on the same stream without clearing. A new one is
    allocated and zero-filled on the stream the library will run on, so the
    fill is ordered before the kernels that rely on it, and the caching
    allocator ties its block to that stream: a buffer it replaces is only
    handed out again to later work on the same stream, after the kernels
    already enqueued there.
    """

    _pool: dict = {}

    @classmethod
    def get(cls, kind: str, nbytes: int, device, stream) -> torch.Tensor:
        stream = _stream_obj(stream)
        key = (kind, torch.device(device).index, stream.cuda_stream)
        ws = cls._pool.get(key)
        if ws is None or ws.numel() < nbytes:
            with torch.cuda.stream(stream):
                ws = torch.zeros(max(nbytes, 4096), dtype=torch.uint8, device=device)
            cls._pool[key] = ws
        return ws


def moe_workspace_clear(ws: torch.Tensor, stream=None) -> None:
    _check("moe_workspace_clear",
           lib().moe_workspace_clear(_ptr(ws, "workspace"), ws.numel() * ws.element_size(),
                                     _stream(stream)))


#: workgroups of moe_hbm_read_probe, one checksum each
HBM_PROBE_GROUPS = 256


def moe_hbm_read_probe(buf: torch.Tensor, checksums: torch.Tensor | None = None,
                       stream=None) -> torch.Tensor:
    """Plain streaming read of buf (the measured HBM read ceiling). Returns
    the per-workgroup XOR checksums [HBM_PROBE_GROUPS] (int32 view of u32)."""
    if checksums is None:
        checksums = torch.empty(HBM_PROBE_GROUPS, dtype=torch.int32, device=buf.device)
    _check("moe_hbm_read_probe",
           lib().moe_hbm_read_probe(_ptr(buf, "buf"), buf.numel() * buf.element_size(),
                                    _ptr(checksums, "checksums"), _stream(stream)))
    return checksums


def moe_route_workspace_bytes(M: int, E: int) -> int:
    return lib().moe_route_workspace_bytes(M, E)


def moe_expert_ffn_workspace_bytes(M: int, H: int, I: int, E: int, k: int) -> int:
    return lib().moe_expert_ffn_workspace_bytes(M, H, I, E, k)


def moe_layer_workspace_bytes(M: int, H: int, I: int, E: int, k: int) -> int:
    return lib().moe_layer_workspace_bytes(M, H, I, E, k)


def lmhead_argmax_workspace_bytes(M: int, V: int) -> int:
    return lib().lmhead_argmax_workspace_bytes(M, V)


def moe_route(x, w_router, k: int, bias=None, *, want_logits=False, out=None,
              workspace=None, stream=None):
    """Router gate GEMV + softmax top-k. Returns (topk_idx, topk_w[, logits])."""
    M, H = x.shape
    E = w_router.shape[0]
    dev = x.device
    idx, w, logits = out if out is not None else (None, None, None)
    if idx is None:
        idx = torch.empty((M, k), dtype=torch.int32, device=dev)
    if w is None:
        w = torch.empty((M, k), dtype=torch.float32, device=dev)
    if want_logits and logits is None:
        logits = torch.empty((M, E), dtype=torch.float32, device=dev)
    st = _stream(stream)
    nbytes = moe_route_workspace_bytes(M, E)
    ws = workspace if workspace is not None else Workspace.get("route", nbytes, dev, stream)
    _check("moe_route", lib().moe_route(
        _ptr(x, "x", _BF16), _ptr(w_router, "w_router", _BF16, (E, H)),
        _ptr(bias, "bias", (torch.float32,), (E,)), M, H, E, k,
        _ptr(idx, "topk_idx", (torch.int32,), (M, k)),
        _ptr(w, "topk_w", (torch.float32,), (M, k)),
        _ptr(logits, "logits", (torch.float32,), (M, E)) if want_logits else None,
        _ptr(ws, "workspace"), ws.numel(), st))
    return (idx, w, logits) if want_logits else (idx, w)


def moe_expert_ffn(x, topk_idx, topk_w, w_gate, w_up, w_down, *, out=None,
                   workspace=None, stream=None):
    """Selected experts' SwiGLU FFN + weighted combine. Returns out [M,H] fp32."""
    M, H = x.shape
    E, I, _ = w_gate.shape
    k = topk_idx.shape[1]
    dev = x.device
    if out is None:
        out = torch.empty((M, H), dtype=torch.float32, device=dev)
    st = _stream(stream)
    nbytes = moe_expert_ffn_workspace_bytes(M, H, I, E, k)
    ws = workspace if workspace is not None else Workspace.get("ffn", nbytes, dev, stream)
    _check("moe_expert_ffn", lib().moe_expert_ffn(
        _ptr(x, "x", _BF16), _ptr(topk_idx, "topk_idx", (torch.int32,), (M, k)),
        _ptr(topk_w, "topk_w", (torch.float32,), (M, k)),
        _ptr(w_gate, "w_gate", _BF16, (E, I, H)), _ptr(w_up, "w_up", _BF16, (E, I, H)),
        _ptr(w_down, "w_down", _BF16, (E, H, I)), M, H, I, E, k,
        _ptr(out, "out", (torch.float32,), (M, H)), _ptr(ws, "workspace"), ws.numel(), st))
    return out


def moe_layer(x, w_router, w_gate, w_up, w_down, k: int, bias=None, *, out=None,
              workspace=None, stream=None):
    """Route + expert FFN in one call. Returns (topk_idx, topk_w, out)."""
    M, H = x.shape
    E, I, _ = w_gate.shape
    dev = x.device
    idx, w, o = out if out is not None else (None, None, None)
    if idx is None:
        idx = torch.empty((M, k), dtype=torch.int32, device=dev)
    if w is None:
        w = torch.empty((M, k), dtype=torch.float32, device=dev)
    if o is None:
        o = torch.empty((M, H), dtype=torch.float32, device=dev)
    st = _stream(stream)
    nbytes = moe_layer_workspace_bytes(M, H, I, E, k)
    ws = workspace if workspace is not None else Workspace.get("layer", nbytes, dev, stream)
    _check("moe_layer", lib().moe_layer(
        _ptr(x, "x", _BF16), _ptr(w_router, "w_router", _BF16, (E, H)),
        _ptr(bias, "bias", (torch.float32,), (E,)),
        _ptr(w_gate, "w_gate", _BF16, (E, I, H)), _ptr(w_up, "w_up", _BF16, (E, I, H)),
        _ptr(w_down, "w_down", _BF16, (E, H, I)), M, H, I, E, k,
        _ptr(idx, "topk_idx", (torch.int32,), (M, k)),
        _ptr(w, "topk_w", (torch.float32,), (M, k)),
        _ptr(o, "out", (torch.float32,), (M, H)), _ptr(ws, "workspace"), ws.numel(), st))
    return idx, w, o


def moe_layer_noalloc(x, w_router, w_gate, w_up, w_down, k: int, bias=None, *, out=None,
                      stream=None):
    """moe_layer with its scratch in the library's own per-GPU array (no
    workspace). Returns (topk_idx, topk_w, out)."""
    M, H = x.shape
    E, I, _ = w_gate.shape
    dev = x.device
    idx, w, o = out if out is not None else (None, None, None)
    if idx is None:
        idx = torch.empty((M, k), dtype=torch.int32, device=dev)
    if w is None:
        w = torch.empty((M, k), dtype=torch.float32, device=dev)
    if o is None:
        o = torch.empty((M, H), dtype=torch.float32, device=dev)
    _check("moe_layer_noalloc", lib().moe_layer_noalloc(
        _ptr(x, "x", _BF16), _ptr(w_router, "w_router", _BF16, (E, H)),
        _ptr(bias, "bias", (torch.float32,), (E,)),
        _ptr(w_gate, "w_gate", _BF16, (E, I, H)), _ptr(w_up, "w_up", _BF16, (E, I, H)),
        _ptr(w_down, "w_down", _BF16, (E, H, I)), M, H, I, E, k,
        _ptr(idx, "topk_idx", (torch.int32,), (M, k)),
        _ptr(w, "topk_w", (torch.float32,), (M, k)),
        _ptr(o, "out", (torch.float32,), (M, H)), _stream(stream)))
    return idx, w, o


def lmhead_argmax(h, w_lm, *, want_max=False, out=None, workspace=None, stream=None):
    """lm_head GEMV + greedy argmax. Returns argmax [M] int32 (, max_logit)."""
    M, H = h.shape
    V = w_lm.shape[0]
    dev = h.device
    am, ml = out if out is not None else (None, None)
    if am is None:
        am = torch.empty(M, dtype=torch.int32, device=dev)
    if want_max and ml is None:
        ml = torch.empty(M, dtype=torch.float32, device=dev)
    st = _stream(stream)
    nbytes = lmhead_argmax_workspace_bytes(M, V)
    ws = workspace if workspace is not None else Workspace.get("lmhead", nbytes, dev, stream)
    _check("lmhead_argmax", lib().lmhead_argmax(
        _ptr(h, "h", _BF16), _ptr(w_lm, "w_lm", _BF16, (V, H)), M, H, V,
        _ptr(am, "argmax", (torch.int32,), (M,)),
        _ptr(ml, "max_logit", (torch.float32,), (M,)) if want_max else None,
        _ptr(ws, "workspace"), ws.numel(), st))
    return (am, ml) if want_max else am


def lmhead_greedy_verify(h, w_lm, tokens, *, want_max=False, out=None, workspace=None,
                         stream=None):
    """lm_head GEMV + greedy argmax + greedy verdict of the chain `tokens`
    ([M] int32: root, then the drafted candidates). Returns (argmax [M] int32,
    accept [2] int32 = (accept length, bonus token)) (, max_logit)."""
    M, H = h.shape
    V = w_lm.shape[0]
    dev = h.device
    am, acc, ml = out if out is not None else (None, None, None)
    if am is None:
        am = torch.empty(M, dtype=torch.int32, device=dev)
    if acc is None:
        acc = torch.empty(2, dtype=torch.int32, device=dev)
    if want_max and ml is None:
        ml = torch.empty(M, dtype=torch.float32, device=dev)
    st = _stream(stream)
    nbytes = lmhead_argmax_workspace_bytes(M, V)
    ws = workspace if workspace is not None else Workspace.get("lmhead", nbytes, dev, stream)
    _check("lmhead_greedy_verify", lib().lmhead_greedy_verify(
        _ptr(h, "h", _BF16), _ptr(w_lm, "w_lm", _BF16, (V, H)),
        _ptr(tokens, "tokens", (torch.int32,), (M,)), M, H, V,
        _ptr(am, "argmax", (torch.int32,), (M,)),
        _ptr(ml, "max_logit", (torch.float32,), (M,)) if want_max else None,
        _ptr(acc, "accept", (torch.int32,), (2,)),
        _ptr(ws, "workspace"), ws.numel(), st))
    return (am, acc, ml) if want_max else (am, acc)


def moe_route_rmsnorm(h, gamma, eps: float, w_router, k: int, bias=None, *, want_logits=False,
                      out=None, workspace=None, stream=None):
    """RMSNorm + router gate GEMV + softmax top-k in one launch.
    Returns (x_norm, topk_idx, topk_w[, logits])."""
    M, H = h.shape
    E = w_router.shape[0]
    dev = h.device
    xn, idx, w, logits = out if out is not None else (None, None, None, None)
    if xn is None:
        xn = torch.empty((M, H), dtype=torch.bfloat16, device=dev)
    if idx is None:
        idx = torch.empty((M, k), dtype=torch.int32, device=dev)
    if w is None:
        w = torch.empty((M, k), dtype=torch.float32, device=dev)
    if want_logits and logits is None:
        logits = torch.empty((M, E), dtype=torch.float32, device=dev)
    st = _stream(stream)
    nbytes = moe_route_workspace_bytes(M, E)
    ws = workspace if workspace is not None else Workspace.get("route", nbytes, dev, stream)
    _check("moe_route_rmsnorm", lib().moe_route_rmsnorm(
        _ptr(h, "h", _BF16), _ptr(gamma, "gamma", _BF16, (H,)), float(eps),
        _ptr(w_router, "w_router", _BF16, (E, H)),
        _ptr(bias, "bias", (torch.float32,), (E,)), M, H, E, k,
        _ptr(xn, "x_norm", _BF16, (M, H)),
        _ptr(idx, "topk_idx", (torch.int32,), (M, k)),
        _ptr(w, "topk_w", (torch.float32,), (M, k)),
        _ptr(logits, "logits", (torch.float32,), (M, E)) if want_logits else None,
        _ptr(ws, "workspace"), ws.numel(), st))
    return (xn, idx, w, logits) if want_logits else (xn, idx, w)


def moe_layer_rmsnorm(h, gamma, eps: float, w_router, w_gate, w_up, w_down, k: int, bias=None,
                      *, out=None, workspace=None, stream=None):
    """RMSNorm + route + expert FFN on the normalised rows.
    Returns (x_norm, topk_idx, topk_w, out)."""
    M, H = h.shape
    E, I, _ = w_gate.shape
    dev = h.device
    xn, idx, w, o = out if out is not None else (None, None, None, None)
    if xn is None:
        xn = torch.empty((M, H), dtype=torch.bfloat16, device=dev)
    if idx is None:
        idx = torch.empty((M, k), dtype=torch.int32, device=dev)
    if w is None:
        w = torch.empty((M, k), dtype=torch.float32, device=dev)
    if o is None:
        o = torch.empty((M, H), dtype=torch.float32, device=dev)
    st = _stream(stream)
    nbytes = moe_layer_workspace_bytes(M, H, I, E, k)
    ws = workspace if workspace is not None else Workspace.get("layer", nbytes, dev, stream)
    _check("moe_layer_rmsnorm", lib().moe_layer_rmsnorm(
        _ptr(h, "h", _BF16), _ptr(gamma, "gamma", _BF16, (H,)), float(eps),
        _ptr(w_router, "w_router", _BF16, (E, H)),
        _ptr(bias, "bias", (torch.float32,), (E,)),
        _ptr(w_gate, "w_gate", _BF16, (E, I, H)), _ptr(w_up, "w_up", _BF16, (E, I, H)),
        _ptr(w_down, "w_down", _BF16, (E, H, I)), M, H, I, E, k,
        _ptr(xn, "x_norm", _BF16, (M, H)),
        _ptr(idx, "topk_idx", (torch.int32,), (M, k)),
        _ptr(w, "topk_w", (torch.float32,), (M, k)),
        _ptr(o, "out", (torch.float32,), (M, H)), _ptr(ws, "workspace"), ws.numel(), st))
    return xn, idx, w, o


def moe_expert_ffn_shared(x, topk_idx, topk_w, w_gate, w_up, w_down, w_gate_shared,
                          w_up_shared, w_down_shared, *, out=None, workspace=None, stream=None):
    """Selected experts' SwiGLU FFN + combine, plus one shared expert with
    weight 1. Returns out [M,H] fp32."""
    M, H = x.shape
    _, k = topk_idx.shape
    E, I, _ = w_gate.shape
    dev = x.device
    o = out if out is not None else torch.empty((M, H), dtype=torch.float32, device=dev)
    st = _stream(stream)
    nbytes = moe_expert_ffn_workspace_bytes(M, H, I, E, k)
    ws = workspace if workspace is not None else Workspace.get("ffn", nbytes, dev, stream)
    _check("moe_expert_ffn_shared", lib().moe_expert_ffn_shared(
        _ptr(x, "x", _BF16), _ptr(topk_idx, "topk_idx", (torch.int32,), (M, k)),
        _ptr(topk_w, "topk_w", (torch.float32,), (M, k)),
        _ptr(w_gate, "w_gate", _BF16, (E, I, H)), _ptr(w_up, "w_up", _BF16, (E, I, H)),
        _ptr(w_down, "w_down", _BF16, (E, H, I)),
        _ptr(w_gate_shared, "w_gate_shared", _BF16, (I, H)),
        _ptr(w_up_shared, "w_up_shared", _BF16, (I, H)),
        _ptr(w_down_shared, "w_down_shared", _BF16, (H, I)), M, H, I, E, k,
        _ptr(o, "out", (torch.float32,), (M, H)), _ptr(ws, "workspace"), ws.numel(), st))
    return o


def moe_layer_shared(x, w_router, w_gate, w_up, w_down, w_gate_shared, w_up_shared,
                     w_down_shared, k: int, bias=None, *, out=None, workspace=None, stream=None):
    """Route + expert FFN with one shared expert. Returns (topk_idx, topk_w, out)."""
    M, H = x.shape
    E, I, _ = w_gate.shape
    dev = x.device
    idx, w, o = out if out is not None else (None, None, None)
    if idx is None:
        idx = torch.empty((M, k), dtype=torch.int32, device=dev)
    if w is None:
        w = torch.empty((M, k), dtype=torch.float32, device=dev)
    if o is None:
        o = torch.empty((M, H), dtype=torch.float32, device=dev)
    st = _stream(stream)
    nbytes = moe_layer_workspace_bytes(M, H, I, E, k)
    ws = workspace if workspace is not None else Workspace.get("layer", nbytes, dev, stream)
    _check("moe_layer_shared", lib().moe_layer_shared(
        _ptr(x, "x", _BF16), _ptr(w_router, "w_router", _BF16, (E, H)),
        _ptr(bias, "bias", (torch.float32,), (E,)),
        _ptr(w_gate, "w_gate", _BF16, (E, I, H)), _ptr(w_up, "w_up", _BF16, (E, I, H)),
        _ptr(w_down, "w_down", _BF16, (E, H, I)),
        _ptr(w_gate_shared, "w_gate_shared", _BF16, (I, H)),
        _ptr(w_up_shared, "w_up_shared", _BF16, (I, H)),
        _ptr(w_down_shared, "w_down_shared", _BF16, (H, I)), M, H, I, E, k,
        _ptr(idx, "topk_idx", (torch.int32,), (M, k)),
        _ptr(w, "topk_w", (torch.float32,), (M, k)),
        _ptr(o, "out", (torch.float32,), (M, H)), _ptr(ws, "workspace"), ws.numel(), st))
    return idx, w, o


_U8 = (torch.uint8,)


def lmhead_argmax_fp8(h, w_lm, w_scale, *, want_max=False, out=None, workspace=None,
                      stream=None):
    """fp8 lm_head (E4M3 codes [V,H] uint8, fp32 scale per row [V]) + greedy
    argmax. Returns argmax [M] int32 (, max_logit)."""
    M, H = h.shape
    V = w_lm.shape[0]
    dev = h.device
    am, ml = out if out is not None else (None, None)
    if am is None:
        am = torch.empty(M, dtype=torch.int32, device=dev)
    if want_max and ml is None:
        ml = torch.empty(M, dtype=torch.float32, device=dev)
    st = _stream(stream)
    nbytes = lmhead_argmax_workspace_bytes(M, V)
    ws = workspace if workspace is not None else Workspace.get("lmhead", nbytes, dev, stream)
    _check("lmhead_argmax_fp8", lib().lmhead_argmax_fp8(
        _ptr(h, "h", _BF16), _ptr(w_lm, "w_lm", _U8, (V, H)),
        _ptr(w_scale, "w_scale", (torch.float32,), (V,)), M, H, V,
        _ptr(am, "argmax", (torch.int32,), (M,)),
        _ptr(ml, "max_logit", (torch.float32,), (M,)) if want_max else None,
        _ptr(ws, "workspace"), ws.numel(), st))
    return (am, ml) if want_max else am


def lmhead_greedy_verify_fp8(h, w_lm, w_scale, tokens, *, want_max=False, out=None,
                             workspace=None, stream=None):
    """fp8 lm_head + greedy argmax + greedy verdict of the chain `tokens`.
    Returns (argmax, accept) (, max_logit)."""
    M, H = h.shape
    V = w_lm.shape[0]
    dev = h.device
    am, acc, ml = out if out is not None else (None, None, None)
    if am is None:
        am = torch.empty(M, dtype=torch.int32, device=dev)
    if acc is None:
        acc = torch.empty(2, dtype=torch.int32, device=dev)
    if want_max and ml is None:
        ml = torch.empty(M, dtype=torch.float32, device=dev)
    st = _stream(stream)
    nbytes = lmhead_argmax_workspace_bytes(M, V)
    ws = workspace if workspace is not None else Workspace.get("lmhead", nbytes, dev, stream)
    _check("lmhead_greedy_verify_fp8", lib().lmhead_greedy_verify_fp8(
        _ptr(h, "h", _BF16), _ptr(w_lm, "w_lm", _U8, (V, H)),
        _ptr(w_scale, "w_scale", (torch.float32,), (V,)),
        _ptr(tokens, "tokens", (torch.int32,), (M,)), M, H, V,
        _ptr(am, "argmax", (torch.int32,), (M,)),
        _ptr(ml, "max_logit", (torch.float32,), (M,)) if want_max else None,
        _ptr(acc, "accept", (torch.int32,), (2,)),
        _ptr(ws, "workspace"), ws.numel(), st))
    return (am, acc, ml) if want_max else (am, acc)


def lmhead_partial_keys(h, w_lm, workspace, *, w_scale=None, stream=None):
    """The lm_head's GEMV phase: each workgroup's per-token winner as a key in
    `workspace` (lmhead_argmax_workspace_bytes(M, V) bytes). With w_scale the
    rows are fp8 codes."""
    M, H = h.shape
    V = w_lm.shape[0]
    st = _stream(stream)
    if w_scale is None:
        _check("lmhead_partial_keys", lib().lmhead_partial_keys(
            _ptr(h, "h", _BF16), _ptr(w_lm, "w_lm", _BF16, (V, H)), M, H, V,
            _ptr(workspace, "workspace"), workspace.numel(), st))
    else:
        _check("lmhead_partial_keys_fp8", lib().lmhead_partial_keys_fp8(
            _ptr(h, "h", _BF16), _ptr(w_lm, "w_lm", _U8, (V, H)),
            _ptr(w_scale, "w_scale", (torch.float32,), (V,)), M, H, V,
            _ptr(workspace, "workspace"), workspace.numel(), st))


def lmhead_merge_keys(M: int, V: int, workspace, *, tokens=None, want_max=False, out=None,
                      stream=None):
    """The lm_head's merge phase over the keys lmhead_partial_keys wrote.
    Returns argmax (, accept with tokens) (, max_logit)."""
    dev = workspace.device
    am, acc, ml = out if out is not None else (None, None, None)
    if am is None:
        am = torch.empty(M, dtype=torch.int32, device=dev)
    if tokens is not None and acc is None:
        acc = torch.empty(2, dtype=torch.int32, device=dev)
    if want_max and ml is None:
        ml = torch.empty(M, dtype=torch.float32, device=dev)
    _check("lmhead_merge_keys", lib().lmhead_merge_keys(
        M, V, _ptr(am, "argmax", (torch.int32,), (M,)),
        _ptr(ml, "max_logit", (torch.float32,), (M,)) if want_max else None,
        _ptr(tokens, "tokens", (torch.int32,), (M,)) if tokens is not None else None,
        _ptr(acc, "accept", (torch.int32,), (2,)) if tokens is not None else None,
        _ptr(workspace, "workspace"), workspace.numel(), _stream(stream)))
    res = (am,) + ((acc,) if tokens is not None else ()) + ((ml,) if want_max else ())
    return res[0] if len(res) == 1 else res


def _fp8_expert_ptrs(E, I, H, w_gate, s_gate, w_up, s_up, w_down, s_down):
    return (_ptr(w_gate, "w_gate", _U8, (E, I, H)), _ptr(s_gate, "s_gate", (torch.float32,), (E, I)),
            _ptr(w_up, "w_up", _U8, (E, I, H)), _ptr(s_up, "s_up", (torch.float32,), (E, I)),
            _ptr(w_down, "w_down", _U8, (E, H, I)), _ptr(s_down, "s_down", (torch.float32,), (E, H)))


def moe_expert_ffn_fp8(x, topk_idx, topk_w, w_gate, s_gate, w_up, s_up, w_down, s_down, *,
                       out=None, workspace=None, stream=None):
    """Selected experts' SwiGLU FFN + combine with fp8 weights (E4M3 codes,
    fp32 row scales). Returns out [M,H] fp32."""
    M, H = x.shape
    _, k = topk_idx.shape
    E, I, _ = w_gate.shape
    dev = x.device
    o = out if out is not None else torch.empty((M, H), dtype=torch.float32, device=dev)
    st = _stream(stream)
    nbytes = moe_expert_ffn_workspace_bytes(M, H, I, E, k)
    ws = workspace if workspace is not None else Workspace.get("ffn", nbytes, dev, stream)
    _check("moe_expert_ffn_fp8", lib().moe_expert_ffn_fp8(
        _ptr(x, "x", _BF16), _ptr(topk_idx, "topk_idx", (torch.int32,), (M, k)),
        _ptr(topk_w, "topk_w", (torch.float32,), (M, k)),
        *_fp8_expert_ptrs(E, I, H, w_gate, s_gate, w_up, s_up, w_down, s_down),
        M, H, I, E, k, _ptr(o, "out", (torch.float32,), (M, H)),
        _ptr(ws, "workspace"), ws.numel(), st))
    return o


def moe_layer_fp8(x, w_router, w_gate, s_gate, w_up, s_up, w_down, s_down, k: int, bias=None,
                  *, out=None, workspace=None, stream=None):
    """Route (bf16 gate) + fp8 expert FFN. Returns (topk_idx, topk_w, out)."""
    M, H = x.shape
    E, I, _ = w_gate.shape
    dev = x.device
    idx, w, o = out if out is not None else (None, None, None)
    if idx is None:
        idx = torch.empty((M, k), dtype=torch.int32, device=dev)
    if w is None:
        w = torch.empty((M, k), dtype=torch.float32, device=dev)
    if o is None:
        o = torch.empty((M, H), dtype=torch.float32, device=dev)
    st = _stream(stream)
    nbytes = moe_layer_workspace_bytes(M, H, I, E, k)
    ws = workspace if workspace is not None else Workspace.get("layer", nbytes, dev, stream)
    _check("moe_layer_fp8", lib().moe_layer_fp8(
        _ptr(x, "x", _BF16), _ptr(w_router, "w_router", _BF16, (E, H)),
        _ptr(bias, "bias", (torch.float32,), (E,)),
        *_fp8_expert_ptrs(E, I, H, w_gate, s_gate, w_up, s_up, w_down, s_down),
        M, H, I, E, k, _ptr(idx, "topk_idx", (torch.int32,), (M, k)),
        _ptr(w, "topk_w", (torch.float32,), (M, k)),
        _ptr(o, "out", (torch.float32,), (M, H)), _ptr(ws, "workspace"), ws.numel(), st))
    return idx, w, o
