"""The layer as its staged entry points on one stream, with preallocated outputs and one
workspace: [moe_rmsnorm ->] moe_route -> moe_permute -> moe_grouped_swiglu (or its MXFP4
form) -> moe_combine.  This is the launch sequence the benchmark times.  Also the upload
of host arrays (bf16 as uint16 bit patterns) to device tensors.  Marshalling only:
buffers come from torch, every step runs in the library's kernels."""
from __future__ import annotations

import numpy as np

from . import moe as M


def config_struct(c) -> "M.moe_config_t":
    """The C config struct of a workload description (any object with d, E, I, k, S,
    router, dtype, bias_on_logits and route_scale)."""
    return M.make_config(c.d, c.E, c.I, c.k, c.S, c.router, c.dtype,
                         bias_on_logits=c.bias_on_logits, route_scale=c.route_scale)


def shared_weights(c, dev: dict):
    """The shared experts' dense weights of an MXFP4 layer (None when S = 0)."""
    if c.S == 0:
        return (None, None, None)
    return (dev["w_gate"], dev["w_up"], dev["w_down"])


def to_dev(a: np.ndarray | None, torch):
    """Host array -> device tensor; bf16 bit patterns (uint16) become torch.bfloat16."""
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a).view(torch.bfloat16).to("cuda")
    return torch.from_numpy(a).to("cuda")


def expert_tensor_to_dev(arr: np.ndarray, torch, chunk: int = 16):
    """Upload a large [E + S, ...] expert tensor chunk by chunk (bounded host temporaries)."""
    dt = torch.bfloat16 if arr.dtype == np.uint16 else torch.float32
    out = torch.empty(arr.shape, dtype=dt, device="cuda")
    for e0 in range(0, arr.shape[0], chunk):
        part = torch.from_numpy(np.ascontiguousarray(arr[e0:e0 + chunk]))
        if arr.dtype == np.uint16:
            part = part.view(torch.bfloat16)
        out[e0:e0 + chunk].copy_(part)
    return out


def packed_scales_to_dev(scales: np.ndarray, torch, stream=None):
    """Upload row-major E8M0 scales [E, N, K/32] and pack them on the device with
    moe_mxfp4_pack_scales (the layout the MXFP4 entry points take)."""
    E, N, KB = scales.shape
    src = to_dev(scales, torch)
    packed = torch.empty(M.moe_mxfp4_scales_bytes(E, N, 32 * KB), dtype=torch.uint8,
                         device="cuda")
    M.moe_mxfp4_pack_scales(E, N, 32 * KB, src, packed, stream)
    torch.cuda.synchronize()
    return packed


def device_inputs(inputs: dict, torch) -> dict:
    """Device copies of a workload's inputs; MXFP4 scales are packed on upload."""
    d = {}
    for k, v in inputs.items():
        if k in ("w_gate", "w_up", "w_down"):
            d[k] = expert_tensor_to_dev(v, torch)
        elif k in ("ws_gate", "ws_up", "ws_down"):
            d[k] = packed_scales_to_dev(v, torch)
        else:
            d[k] = to_dev(v, torch)
    return d


class StagedRunner:
    """One layer's staged launch sequence on device tensors ``dev`` (x, w_router,
    sel_bias, logit_offset, w_gate / w_up / w_down, or the MXFP4 codes and packed scales
    wq_* / ws_* with the shared experts' dense weights, and norm_gain for pre-norm
    layers, whose x is the raw hidden state)."""

    def __init__(self, c, dev: dict, torch):
        self.c, self.dev, self.torch = c, dev, torch
        self.cfg = config_struct(c)
        T = dev["x"].shape[0]
        self.T = T
        A, G = c.k + c.S, c.E + c.S
        R = T * A
        self.nws = M.moe_workspace_size(self.cfg, T)
        e = dict(device="cuda")
        self.ws = torch.empty(max(self.nws, 256), dtype=torch.uint8, **e)
        self.idx = torch.empty((T, c.k), dtype=torch.int32, **e)
        self.w = torch.empty((T, A), dtype=torch.float32, **e)
        self.counts = torch.empty((G,), dtype=torch.int32, **e)
        self.offsets = torch.empty((G + 1,), dtype=torch.int32, **e)
        self.row_token = torch.empty((R,), dtype=torch.int32, **e)
        self.slot_row = torch.empty((R,), dtype=torch.int32, **e)
        self.y_rows = torch.empty((R, c.d), dtype=torch.float32, **e)
        self.out = torch.empty((T, c.d), dtype=torch.float32, **e)
        self.xn = torch.empty_like(dev["x"]) if c.prenorm else None

    def step(self, stream, ev=None, residual=None):
        """Enqueue one layer on ``stream``; ``ev`` (five events) brackets the stages:
        route (with the pre-norm), permute, grouped SwiGLU, combine."""
        d, c, T, cfg = self.dev, self.c, self.T, self.cfg
        if ev is not None:
            ev[0].record(stream)
        x = d["x"]
        if c.prenorm:
            M.moe_rmsnorm(cfg, T, x, d["norm_gain"], c.norm_eps, c.norm_zero_centred,
                          self.xn, stream)
            x = self.xn
        M.moe_route(cfg, T, x, d["w_router"], d.get("sel_bias"), d.get("logit_offset"),
                    self.idx, self.w, self.ws, self.nws, stream)
        if ev is not None:
            ev[1].record(stream)
        M.moe_permute(cfg, T, self.idx, self.counts, self.offsets, self.row_token,
                      self.slot_row, self.ws, self.nws, stream)
        if ev is not None:
            ev[2].record(stream)
        if c.weight_format == "mxfp4":
            M.moe_grouped_swiglu_mxfp4(cfg, T, x, self.offsets, self.row_token,
                                       d["wq_gate"], d["ws_gate"], d["wq_up"], d["ws_up"],
                                       d["wq_down"], d["ws_down"], *shared_weights(c, d),
                                       self.y_rows, self.ws, self.nws, stream)
        else:
            M.moe_grouped_swiglu(cfg, T, x, self.offsets, self.row_token, d["w_gate"],
                                 d["w_up"], d["w_down"], self.y_rows, self.ws, self.nws,
                                 stream)
        if ev is not None:
            ev[3].record(stream)
        M.moe_combine(cfg, T, self.y_rows, self.slot_row, self.w, residual, self.out, stream)
        if ev is not None:
            ev[4].record(stream)
