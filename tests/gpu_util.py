"""Helpers of the GPU tests and the bench: host arrays <-> device tensors, config
structs, and calls of the library through its C ABI.  Marshalling only.  The staged
launch sequence (StagedRunner) lives in the package."""
from __future__ import annotations

import numpy as np

import sparse_mixture_experts_fp32_amd as M
from sparse_mixture_experts_fp32_amd.staged import (  # noqa: F401
    StagedRunner, config_struct, device_inputs, expert_tensor_to_dev, packed_scales_to_dev,
    shared_weights, to_dev)


cfg_struct = config_struct


def packed_scale_order(scales: np.ndarray) -> np.ndarray:
    """The packed-record order of row-major scales [E, N, K/32], by numpy reshapes:
    record (e, 64-row block, 8-block run of K) holds 64 rows x 8 bytes, zero-padded."""
    E, N, KB = scales.shape
    KR = -(-KB // 8)
    pad = np.zeros((E, N, 8 * KR), np.uint8)
    pad[:, :, :KB] = scales
    return pad.reshape(E, N // 64, 64, KR, 8).transpose(0, 1, 3, 2, 4).reshape(-1)


def workspace(cfg, T, torch):
    n = M.moe_workspace_size(cfg, T)
    return torch.empty(max(n, 256), dtype=torch.uint8, device="cuda"), n




def run_forward(c, dev: dict, torch, residual=None, ws=None):
    """moe_forward (moe_forward_rmsnorm for pre-norm workloads, whose x is the raw hidden
    state) on device tensors; returns (out, topk_idx, counts) device tensors."""
    cfg = cfg_struct(c)
    T = dev["x"].shape[0]
    if ws is None:
        ws = workspace(cfg, T, torch)
    buf, n = ws
    out = torch.empty((T, c.d), dtype=torch.float32, device="cuda")
    idx = torch.empty((T, c.k), dtype=torch.int32, device="cuda")
    counts = torch.empty((c.E + c.S,), dtype=torch.int32, device="cuda")
    if c.weight_format == "mxfp4":
        sh = shared_weights(c, dev)
        M.moe_forward_mxfp4(cfg, T, dev["x"], dev["w_router"], dev.get("sel_bias"),
                            dev.get("logit_offset"), dev["wq_gate"], dev["ws_gate"],
                            dev["wq_up"], dev["ws_up"], dev["wq_down"], dev["ws_down"], *sh,
                            residual, out, idx, counts, buf, n)
    elif c.prenorm:
        M.moe_forward_rmsnorm(cfg, T, dev["x"], dev["norm_gain"], c.norm_eps,
                              c.norm_zero_centred, dev["w_router"], dev.get("sel_bias"),
                              dev.get("logit_offset"), dev["w_gate"], dev["w_up"],
                              dev["w_down"], residual, out, idx, counts, buf, n)
    else:
        M.moe_forward(cfg, T, dev["x"], dev["w_router"], dev.get("sel_bias"),
                      dev.get("logit_offset"), dev["w_gate"], dev["w_up"], dev["w_down"],
                      residual, out, idx, counts, buf, n)
    return out, idx, counts


def host_grouping(idx: np.ndarray, E: int, S: int):
    """Rows grouped by expert from a host-side selection (ascending token order within a
    group, shared experts' groups last): the layout the library's permute produces."""
    T, k = idx.shape
    A = k + S
    flat = idx.ravel()
    tok = np.repeat(np.arange(T), k)
    slot = np.tile(np.arange(k), T)
    order = np.argsort(flat, kind="stable")           # by expert, then token
    counts = np.concatenate([np.bincount(flat, minlength=E), np.full(S, T)])
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    row_token = np.concatenate([tok[order]] + [np.arange(T)] * S).astype(np.int32)
    slot_row = np.empty((T, A), np.int32)
    slot_row[tok[order], slot[order]] = np.arange(T * k)
    for s in range(S):
        slot_row[:, k + s] = T * k + s * T + np.arange(T)
    return counts.astype(np.int32), offsets, row_token, slot_row
