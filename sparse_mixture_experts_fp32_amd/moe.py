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
    _check(load_library().moe_route(ctypes.byref(cfg), T, _ptr(x), _ptr(w_router),
                                    _ptr(sel_bias), _ptr(logit_offset), _ptr(topk_idx),
                                    _ptr(weights), _ptr(ws), ws_bytes, _stream(stream)))


def moe_permute(cfg, T, topk_idx, counts, offsets, row_token, slot_row, ws, ws_bytes,
                stream=None):
    _check(load_library().moe_permute(ctypes.byref(cfg), T, _ptr(topk_idx), _ptr(counts),
                                      _ptr(offsets), _ptr(row_token), _ptr(slot_row),
                                      _ptr(ws), ws_bytes, _stream(stream)))


def moe_grouped_swiglu(cfg, T, x, offsets, row_token, w_gate, w_up, w_down, y_rows, ws,
                       ws_bytes, stream=None):
    _check(load_library().moe_grouped_swiglu(ctypes.byref(cfg), T, _ptr(x), _ptr(offsets),
                                             _ptr(row_token), _ptr(w_gate), _ptr(w_up),
                                             _ptr(w_down), _ptr(y_rows), _ptr(ws), ws_bytes,
                                             _stream(stream)))


def moe_combine(cfg, T, y_rows, slot_row, weights, residual, out, stream=None):
    _check(load_library().moe_combine(ctypes.byref(cfg), T, _ptr(y_rows), _ptr(slot_row),
                                      _ptr(weights), _ptr(residual), _ptr(out),
                                      _stream(stream)))


def moe_forward(cfg, T, x, w_router, sel_bias, logit_offset, w_gate, w_up, w_down, residual,
                out, topk_idx_out, counts_out, ws, ws_bytes, stream=None):
    _check(load_library().moe_forward(ctypes.byref(cfg), T, _ptr(x), _ptr(w_router),
                                      _ptr(sel_bias), _ptr(logit_offset), _ptr(w_gate),
                                      _ptr(w_up), _ptr(w_down), _ptr(residual), _ptr(out),
                                      _ptr(topk_idx_out), _ptr(counts_out), _ptr(ws),
                                      ws_bytes, _stream(stream)))


def moe_rmsnorm(cfg, T, x, gain, eps, zero_centred, y, stream=None):
    _check(load_library().moe_rmsnorm(ctypes.byref(cfg), T, _ptr(x), _ptr(gain), float(eps),
                                      int(zero_centred), _ptr(y), _stream(stream)))


def moe_forward_rmsnorm(cfg, T, x, norm_gain, eps, zero_centred, w_router, sel_bias,
                        logit_offset, w_gate, w_up, w_down, residual, out, topk_idx_out,
                        counts_out, ws, ws_bytes, stream=None):
    _check(load_library().moe_forward_rmsnorm(
        ctypes.byref(cfg), T, _ptr(x), _ptr(norm_gain), float(eps), int(zero_centred),
        _ptr(w_router), _ptr(sel_bias), _ptr(logit_offset), _ptr(w_gate), _ptr(w_up),
        _ptr(w_down), _ptr(residual), _ptr(out), _ptr(topk_idx_out), _ptr(counts_out),
        _ptr(ws), ws_bytes, _stream(stream)))


def moe_mxfp4_scales_bytes(E: int, N: int, K: int) -> int:
    out = ctypes.c_size_t(0)
    _check(load_library().moe_mxfp4_scales_bytes(E, N, K, ctypes.byref(out)))
    return out.value


def moe_mxfp4_pack_scales(E, N, K, scales, packed, stream=None):
    _check(load_library().moe_mxfp4_pack_scales(E, N, K, _ptr(scales), _ptr(packed),
                                                _stream(stream)))


def moe_grouped_swiglu_mxfp4(cfg, T, x, offsets, row_token, wq_gate, ws_gate, wq_up, ws_up,
                             wq_down, ws_down, w_gate_shared, w_up_shared, w_down_shared,
                             y_rows, ws, ws_bytes, stream=None):
    _check(load_library().moe_grouped_swiglu_mxfp4(
        ctypes.byref(cfg), T, _ptr(x), _ptr(offsets), _ptr(row_token), _ptr(wq_gate),
        _ptr(ws_gate), _ptr(wq_up), _ptr(ws_up), _ptr(wq_down), _ptr(ws_down),
        _ptr(w_gate_shared), _ptr(w_up_shared), _ptr(w_down_shared), _ptr(y_rows),
        _ptr(ws), ws_bytes, _stream(stream)))


def moe_forward_mxfp4(cfg, T, x, w_router, sel_bias, logit_offset, wq_gate, ws_gate, wq_up,
                      ws_up, wq_down, ws_down, w_gate_shared, w_up_shared, w_down_shared,
                      residual, out, topk_idx_out, counts_out, ws, ws_bytes, stream=None):
    _check(load_library().moe_forward_mxfp4(
        ctypes.byref(cfg), T, _ptr(x), _ptr(w_router), _ptr(sel_bias), _ptr(logit_offset),
        _ptr(wq_gate), _ptr(ws_gate), _ptr(wq_up), _ptr(ws_up), _ptr(wq_down), _ptr(ws_down),
        _ptr(w_gate_shared), _ptr(w_up_shared), _ptr(w_down_shared), _ptr(residual),
        _ptr(out), _ptr(topk_idx_out), _ptr(counts_out), _ptr(ws), ws_bytes,
        _stream(stream)))
