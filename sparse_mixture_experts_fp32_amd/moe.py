"""Python binding of libmoe.so (the MI355X mixture-of-experts layer).

Argument marshalling only: every step of the layer runs in the library's HIP kernels.
Tensors are passed as device pointers (torch tensors' ``data_ptr()`` or plain ints),
streams as ``hipStream_t`` handles (default: torch's current stream).  The functions
have the C ABI's names and argument order; a non-OK status raises ``MoEError``.
"""
from __future__ import annotations

import ctypes
import os
import re

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe.so")
HEADER_PATH = os.path.join(os.path.dirname(_PKG), "include", "moe.h")

MOE_OK, MOE_ERR_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = range(5)
MOE_ROUTER_SOFTMAX_TOPK, MOE_ROUTER_SIGMOID_SHARED = 0, 1
MOE_F32, MOE_BF16 = 0, 1


class MoEError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


class moe_config_t(ctypes.Structure):
    _fields_ = [("d_model", ctypes.c_int32), ("n_experts", ctypes.c_int32),
                ("d_ff", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("n_shared", ctypes.c_int32), ("router", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("bias_on_logits", ctypes.c_int32),
                ("route_scale", ctypes.c_float)]


def make_config(d_model, n_experts, d_ff, top_k, n_shared, router, dtype,
                bias_on_logits=False, route_scale=None) -> moe_config_t:
    """router: "softmax" | "sigmoid" (or the enum); dtype: "f32" | "bf16" (or the enum).
    route_scale defaults to k + S for the sigmoid router and 1 for softmax."""
    r = {"softmax": MOE_ROUTER_SOFTMAX_TOPK, "sigmoid": MOE_ROUTER_SIGMOID_SHARED}.get(
        router, router)
    dt = {"f32": MOE_F32, "bf16": MOE_BF16}.get(dtype, dtype)
    if route_scale is None:
        route_scale = float(top_k + n_shared) if r == MOE_ROUTER_SIGMOID_SHARED else 1.0
    return moe_config_t(int(d_model), int(n_experts), int(d_ff), int(top_k), int(n_shared),
                        int(r), int(dt), int(bool(bias_on_logits)), float(route_scale))


_lib = None
ARGTYPES: dict = {}   # entry point -> number of C parameters bound (set by load_library)


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libmoe.so; raises if it has not been built (there is no fallback path)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           "`python -m sparse_mixture_experts_fp32_amd.build`")
    # The tensors handed to the library come from torch's HIP runtime; load that
    # runtime first so the library binds to the same one rather than to another copy.
    try:
        import torch  # noqa: F401
    except ImportError:  # pragma: no cover - torch-free use of the C ABI
        pass
    lib = ctypes.CDLL(path)
    P, I64, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t
    CFG = ctypes.POINTER(moe_config_t)
    lib.moe_status_str.restype = ctypes.c_char_p
    lib.moe_status_str.argtypes = [ctypes.c_int]
    sigs = {
        "moe_workspace_size": [CFG, I64, ctypes.POINTER(SZ)],
        "moe_route": [CFG, I64, P, P, P, P, P, P, P, SZ, P],
        "moe_permute": [CFG, I64, P, P, P, P, P, P, SZ, P],
        "moe_grouped_swiglu": [CFG, I64, P, P, P, P, P, P, P, P, SZ, P],
        "moe_combine": [CFG, I64, P, P, P, P, P, P],
        "moe_forward": [CFG, I64, P, P, P, P, P, P, P, P, P, P, P, P, SZ, P],
        "moe_rmsnorm": [CFG, I64, P, P, ctypes.c_float, ctypes.c_int32, P, P],
        "moe_grouped_swiglu_mxfp4": [CFG, I64, P, P, P, P, P, P, P, P, P, P, P, P, P, P, SZ,
                                     P],
        "moe_forward_mxfp4": [CFG, I64, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P, P,
                              SZ, P],
        "moe_forward_rmsnorm": [CFG, I64, P, P, ctypes.c_float, ctypes.c_int32, P, P, P, P,
                                P, P, P, P, P, P, P, SZ, P],
        "moe_mxfp4_scales_bytes": [I64, I64, I64, ctypes.POINTER(SZ)],
        "moe_mxfp4_pack_scales": [I64, I64, I64, P, P, P],
        "moe_forward_static": [CFG, I64, P, P, P, P, P, P, P, P, P, P, P, P],
    }
    global ARGTYPES
    ARGTYPES = {name: len(args) for name, args in sigs.items()}
    for name, args in sigs.items():
        fn = getattr(lib, name)
        fn.restype = ctypes.c_int
        fn.argtypes = args
    _lib = lib
    return lib


def header_param_counts(path: str = HEADER_PATH) -> dict:
    """Number of parameters of each function include/moe.h declares."""
    src = re.sub(r"/\*.*?\*/", "", open(path).read(), flags=re.S)
    out = {}
    for m in re.finditer(r"(moe_\w+)\s*\(([^;{]*?)\)\s*;", src, re.S):
        params = m.group(2).strip()
        out[m.group(1)] = 0 if params in ("", "void") else params.count(",") + 1
    return out


def header_functions(path: str = HEADER_PATH) -> list[str]:
    """Names of the functions include/moe.h declares."""
    src = open(path).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(moe_\w+)\s*\(", src, re.M)))


def _ptr(t):
    """Device address of a tensor argument (None passes NULL; an int is taken as an address
    the caller vouches for).  A tensor must live on a GPU and be contiguous: the kernels
    read every buffer as dense row-major device memory, and a host address would fault."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise ValueError(f"expected a GPU tensor, got one on {t.device}")
    if not t.is_contiguous():
        raise ValueError("expected a contiguous tensor (dense row-major)")
    return t.data_ptr()


# Element types of tensor arguments: "layer" is the config's dtype (bf16 or f32).
_KINDS = {"f32": "float32", "i32": "int32", "u8": "uint8", "bf16": "bfloat16"}


def _arg(t, what: str, kind: str, numel: int, cfg=None):
    """``_ptr`` of tensor argument ``what`` after checking that its element type is
    ``kind`` and that it holds at least ``numel`` elements (the extent the header gives
    for this config and token count); raises ValueError otherwise.  Ints and None pass
    unchecked, as in ``_ptr``."""
    if t is None or isinstance(t, int):
        return _ptr(t)
    import torch
    if kind == "layer":
        kind = "bf16" if cfg.dtype == MOE_BF16 else "f32"
    want = getattr(torch, _KINDS[kind])
    if t.dtype != want:
        raise ValueError(f"{what}: expected {want}, got {t.dtype}")
    if t.numel() < numel:
        raise ValueError(f"{what}: holds {t.numel()} elements, the call reads {numel}")
    return _ptr(t)


def _ws(t, ws_bytes: int):
    """Workspace pointer: any element type, at least ``ws_bytes`` bytes."""
    if t is None or isinstance(t, int):
        return _ptr(t)
    if t.numel() * t.element_size() < ws_bytes:
        raise ValueError(f"ws: {t.numel() * t.element_size()} bytes, ws_bytes says "
                         f"{ws_bytes}")
    return _ptr(t)


class _Dims:
    """Extents of a call's tensors (include/moe.h): T tokens, d, E, S, I, k, the k + S
    active experts per token (A), E + S groups (G), T A grouped rows (R) and the router
    rows (NR: E + S for the sigmoid router, E for softmax)."""

    def __init__(self, cfg, T):
        self.T, self.d, self.E, self.S = int(T), cfg.d_model, cfg.n_experts, cfg.n_shared
        self.I, self.k = cfg.d_ff, cfg.top_k
        self.A, self.G = self.k + self.S, self.E + self.S
        self.R = self.T * self.A
        self.NR = self.G if cfg.router == MOE_ROUTER_SIGMOID_SHARED else self.E


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status: int):
    if status != MOE_OK:
        msg = load_library().moe_status_str(status).decode()
        raise MoEError(status, msg)


def status_str(status: int) -> str:
    return load_library().moe_status_str(status).decode()


def moe_workspace_size(cfg: moe_config_t, T: int) -> int:
    out = ctypes.c_size_t(0)
    _check(load_library().moe_workspace_size(ctypes.byref(cfg), T, ctypes.byref(out)))
    return out.value


def moe_route(cfg, T, x, w_router, sel_bias, logit_offset, topk_idx, weights, ws, ws_bytes,
              stream=None):
    m = _Dims(cfg, T)
    _check(load_library().moe_route(
        ctypes.byref(cfg), T, _arg(x, "x", "layer", m.T * m.d, cfg),
        _arg(w_router, "w_router", "layer", m.NR * m.d, cfg),
        _arg(sel_bias, "sel_bias", "f32", m.E), _arg(logit_offset, "logit_offset", "f32", m.E),
        _arg(topk_idx, "topk_idx", "i32", m.T * m.k),
        _arg(weights, "weights", "f32", m.T * m.A), _ws(ws, ws_bytes), ws_bytes,
        _stream(stream)))


def moe_permute(cfg, T, topk_idx, counts, offsets, row_token, slot_row, ws, ws_bytes,
                stream=None):
    m = _Dims(cfg, T)
    _check(load_library().moe_permute(
        ctypes.byref(cfg), T, _arg(topk_idx, "topk_idx", "i32", m.T * m.k),
        _arg(counts, "counts", "i32", m.G), _arg(offsets, "offsets", "i32", m.G + 1),
        _arg(row_token, "row_token", "i32", m.R), _arg(slot_row, "slot_row", "i32", m.R),
        _ws(ws, ws_bytes), ws_bytes, _stream(stream)))


def _experts(cfg, m, w_gate, w_up, w_down, n):
    """Dense expert weights of n experts: gate/up [n, I, d], down [n, d, I]."""
    return (_arg(w_gate, "w_gate", "layer", n * m.I * m.d, cfg),
            _arg(w_up, "w_up", "layer", n * m.I * m.d, cfg),
            _arg(w_down, "w_down", "layer", n * m.d * m.I, cfg))


def moe_grouped_swiglu(cfg, T, x, offsets, row_token, w_gate, w_up, w_down, y_rows, ws,
                       ws_bytes, stream=None):
    m = _Dims(cfg, T)
    _check(load_library().moe_grouped_swiglu(
        ctypes.byref(cfg), T, _arg(x, "x", "layer", m.T * m.d, cfg),
        _arg(offsets, "offsets", "i32", m.G + 1), _arg(row_token, "row_token", "i32", m.R),
        *_experts(cfg, m, w_gate, w_up, w_down, m.G), _arg(y_rows, "y_rows", "f32", m.R * m.d),
        _ws(ws, ws_bytes), ws_bytes, _stream(stream)))


def moe_combine(cfg, T, y_rows, slot_row, weights, residual, out, stream=None):
    m = _Dims(cfg, T)
    _check(load_library().moe_combine(
        ctypes.byref(cfg), T, _arg(y_rows, "y_rows", "f32", m.R * m.d),
        _arg(slot_row, "slot_row", "i32", m.R), _arg(weights, "weights", "f32", m.T * m.A),
        _arg(residual, "residual", "f32", m.T * m.d), _arg(out, "out", "f32", m.T * m.d),
        _stream(stream)))


def _forward_tail(cfg, m, residual, out, topk_idx_out, counts_out):
    return (_arg(residual, "residual", "f32", m.T * m.d), _arg(out, "out", "f32", m.T * m.d),
            _arg(topk_idx_out, "topk_idx_out", "i32", m.T * m.k),
            _arg(counts_out, "counts_out", "i32", m.G))


def moe_forward(cfg, T, x, w_router, sel_bias, logit_offset, w_gate, w_up, w_down, residual,
                out, topk_idx_out, counts_out, ws, ws_bytes, stream=None):
    m = _Dims(cfg, T)
    _check(load_library().moe_forward(
        ctypes.byref(cfg), T, _arg(x, "x", "layer", m.T * m.d, cfg),
        _arg(w_router, "w_router", "layer", m.NR * m.d, cfg),
        _arg(sel_bias, "sel_bias", "f32", m.E), _arg(logit_offset, "logit_offset", "f32", m.E),
        *_experts(cfg, m, w_gate, w_up, w_down, m.G),
        *_forward_tail(cfg, m, residual, out, topk_idx_out, counts_out),
        _ws(ws, ws_bytes), ws_bytes, _stream(stream)))


def moe_forward_static(cfg, T, x, w_router, sel_bias, logit_offset, w_gate, w_up, w_down,
                       residual, out, topk_idx_out, counts_out, stream=None):
    """moe_forward with the library's static device scratch instead of a workspace (for
    callers that cannot allocate; at most MOE_STATIC_SCRATCH_BYTES of workspace)."""
    m = _Dims(cfg, T)
    _check(load_library().moe_forward_static(
        ctypes.byref(cfg), T, _arg(x, "x", "layer", m.T * m.d, cfg),
        _arg(w_router, "w_router", "layer", m.NR * m.d, cfg),
        _arg(sel_bias, "sel_bias", "f32", m.E), _arg(logit_offset, "logit_offset", "f32", m.E),
        *_experts(cfg, m, w_gate, w_up, w_down, m.G),
        *_forward_tail(cfg, m, residual, out, topk_idx_out, counts_out), _stream(stream)))


MOE_STATIC_SCRATCH_BYTES = 64 << 20


def moe_rmsnorm(cfg, T, x, gain, eps, zero_centred, y, stream=None):
    m = _Dims(cfg, T)
    _check(load_library().moe_rmsnorm(
        ctypes.byref(cfg), T, _arg(x, "x", "layer", m.T * m.d, cfg),
        _arg(gain, "gain", "layer", m.d, cfg), float(eps), int(zero_centred),
        _arg(y, "y", "layer", m.T * m.d, cfg), _stream(stream)))


def moe_forward_rmsnorm(cfg, T, x, norm_gain, eps, zero_centred, w_router, sel_bias,
                        logit_offset, w_gate, w_up, w_down, residual, out, topk_idx_out,
                        counts_out, ws, ws_bytes, stream=None):
    m = _Dims(cfg, T)
    _check(load_library().moe_forward_rmsnorm(
        ctypes.byref(cfg), T, _arg(x, "x", "layer", m.T * m.d, cfg),
        _arg(norm_gain, "norm_gain", "layer", m.d, cfg), float(eps), int(zero_centred),
        _arg(w_router, "w_router", "layer", m.NR * m.d, cfg),
        _arg(sel_bias, "sel_bias", "f32", m.E), _arg(logit_offset, "logit_offset", "f32", m.E),
        *_experts(cfg, m, w_gate, w_up, w_down, m.G),
        *_forward_tail(cfg, m, residual, out, topk_idx_out, counts_out),
        _ws(ws, ws_bytes), ws_bytes, _stream(stream)))


def moe_mxfp4_scales_bytes(E: int, N: int, K: int) -> int:
    out = ctypes.c_size_t(0)
    _check(load_library().moe_mxfp4_scales_bytes(E, N, K, ctypes.byref(out)))
    return out.value


def moe_mxfp4_pack_scales(E, N, K, scales, packed, stream=None):
    nbytes = moe_mxfp4_scales_bytes(E, N, K)
    _check(load_library().moe_mxfp4_pack_scales(
        E, N, K, _arg(scales, "scales", "u8", E * N * (K // 32)),
        _arg(packed, "packed", "u8", nbytes), _stream(stream)))


def _mxfp4(cfg, m, wq_gate, ws_gate, wq_up, ws_up, wq_down, ws_down, wg_s, wu_s, wd_s):
    """MXFP4 routed experts' codes and packed scales, then the shared experts' bf16
    weights [S, I, d] / [S, d, I]."""
    sgu = moe_mxfp4_scales_bytes(m.E, m.I, m.d)
    sdn = moe_mxfp4_scales_bytes(m.E, m.d, m.I)
    n = m.E * m.I * m.d // 2
    return (_arg(wq_gate, "wq_gate", "u8", n), _arg(ws_gate, "ws_gate", "u8", sgu),
            _arg(wq_up, "wq_up", "u8", n), _arg(ws_up, "ws_up", "u8", sgu),
            _arg(wq_down, "wq_down", "u8", n), _arg(ws_down, "ws_down", "u8", sdn),
            _arg(wg_s, "w_gate_shared", "bf16", m.S * m.I * m.d),
            _arg(wu_s, "w_up_shared", "bf16", m.S * m.I * m.d),
            _arg(wd_s, "w_down_shared", "bf16", m.S * m.d * m.I))


def moe_grouped_swiglu_mxfp4(cfg, T, x, offsets, row_token, wq_gate, ws_gate, wq_up, ws_up,
                             wq_down, ws_down, w_gate_shared, w_up_shared, w_down_shared,
                             y_rows, ws, ws_bytes, stream=None):
    m = _Dims(cfg, T)
    _check(load_library().moe_grouped_swiglu_mxfp4(
        ctypes.byref(cfg), T, _arg(x, "x", "layer", m.T * m.d, cfg),
        _arg(offsets, "offsets", "i32", m.G + 1), _arg(row_token, "row_token", "i32", m.R),
        *_mxfp4(cfg, m, wq_gate, ws_gate, wq_up, ws_up, wq_down, ws_down, w_gate_shared,
                w_up_shared, w_down_shared),
        _arg(y_rows, "y_rows", "f32", m.R * m.d), _ws(ws, ws_bytes), ws_bytes,
        _stream(stream)))


def moe_forward_mxfp4(cfg, T, x, w_router, sel_bias, logit_offset, wq_gate, ws_gate, wq_up,
                      ws_up, wq_down, ws_down, w_gate_shared, w_up_shared, w_down_shared,
                      residual, out, topk_idx_out, counts_out, ws, ws_bytes, stream=None):
    m = _Dims(cfg, T)
    _check(load_library().moe_forward_mxfp4(
        ctypes.byref(cfg), T, _arg(x, "x", "layer", m.T * m.d, cfg),
        _arg(w_router, "w_router", "layer", m.NR * m.d, cfg),
        _arg(sel_bias, "sel_bias", "f32", m.E), _arg(logit_offset, "logit_offset", "f32", m.E),
        *_mxfp4(cfg, m, wq_gate, ws_gate, wq_up, ws_up, wq_down, ws_down, w_gate_shared,
                w_up_shared, w_down_shared),
        *_forward_tail(cfg, m, residual, out, topk_idx_out, counts_out),
        _ws(ws, ws_bytes), ws_bytes, _stream(stream)))
