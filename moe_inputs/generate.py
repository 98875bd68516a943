"""Seeded synthetic inputs for the mixture-of-experts layer.

This module is shared by the CPU oracle's tests and by the GPU path's tests and bench; it
holds none of the layer's arithmetic.  It only draws numbers:

* every tensor is drawn from its own counter-keyed stream:
  ``SeedSequence(seed, spawn_key=(tensor id, block))`` feeding an SFC64 generator, so any
  expert (or any 1,024-token block of x) can be regenerated on its own, in any order;
* values are ``std * standard_normal()`` in float32; for bf16 workloads they are then
  rounded to bf16 (round to nearest, ties to even) and kept as raw uint16 bit patterns;
* the selection bias and the Zipf logit offset stay float32.

Layouts (row-major, contiguous):
  x          [T, d]
  w_router   [NR, d]      (sigmoid: NR = E + S, shared experts' rows last; softmax:
                           NR = E, its shared experts are ungated)
  sel_bias   [E]          (sigmoid router only)
  logit_off  [E]          (Zipf-skewed workload only)
  norm_gain  [d]          (pre-norm workloads only; RMSNorm gains in the layer dtype)
  w_gate     [E + S, I, d]
  w_up       [E + S, I, d]
  w_down     [E + S, d, I]
MXFP4 workloads (routed experts only; ``w_*`` then hold the S shared experts):
  wq_gate, wq_up [E, I, d/2] uint8 codes;  ws_gate, ws_up [E, I, d/32] uint8 scales
  wq_down        [E, d, I/2] uint8 codes;  ws_down        [E, d, I/32] uint8 scales
"""
from __future__ import annotations

import json
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from .configs import MoEConfig

TENSOR_IDS = {"x": 1, "w_router": 2, "sel_bias": 3, "zipf_rank": 4,
              "w_gate": 5, "w_up": 6, "w_down": 7, "norm_gain": 8}
X_BLOCK = 1024  # tokens per x stream
_CALIB_FILE = os.path.join(os.path.dirname(__file__), "zipf_calibration.json")


def default_threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _rng(seed: int, tensor: str, block: int) -> np.random.Generator:
    ss = np.random.SeedSequence(seed, spawn_key=(TENSOR_IDS[tensor], block))
    return np.random.Generator(np.random.SFC64(ss))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); return the uint16 bits."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    r = (u >> np.uint32(16)) & np.uint32(1)
    r += np.uint32(0x7FFF)
    r += u
    r >>= np.uint32(16)
    return r.astype(np.uint16)


def _draw(rng: np.random.Generator, shape, std: float, dtype: str) -> np.ndarray:
    v = rng.standard_normal(size=shape, dtype=np.float32)
    np.multiply(v, np.float32(std), out=v)
    return f32_to_bf16_bits(v) if dtype == "bf16" else v


def storage_dtype(cfg: MoEConfig):
    return np.uint16 if cfg.dtype == "bf16" else np.float32


# ----------------------------------------------------------------------------- x, router
def make_x(cfg: MoEConfig, T: int | None = None) -> np.ndarray:
    """Hidden states x [T, d]; tokens are drawn in blocks of 1,024 from separate streams."""
    T = cfg.T if T is None else T
    out = np.empty((T, cfg.d), storage_dtype(cfg))
    nblk = (T + X_BLOCK - 1) // X_BLOCK

    def one(b):
        t0, t1 = b * X_BLOCK, min(T, (b + 1) * X_BLOCK)
        # Each block always draws a full X_BLOCK rows so that a prefix of a larger batch
        # is the same batch.
        v = _draw(_rng(cfg.seed, "x", b), (X_BLOCK, cfg.d), cfg.x_std, cfg.dtype)
        out[t0:t1] = v[: t1 - t0]

    if nblk == 1:
        one(0)
    else:
        with ThreadPoolExecutor(min(nblk, default_threads())) as ex:
            list(ex.map(one, range(nblk)))
    return out


def make_w_router(cfg: MoEConfig) -> np.ndarray:
    return _draw(_rng(cfg.seed, "w_router", 0), (cfg.router_rows, cfg.d), cfg.w_std,
                 cfg.dtype)


def make_norm_gain(cfg: MoEConfig) -> np.ndarray | None:
    """RMSNorm gains [d] in the layer dtype for pre-norm workloads: stored g ~ N(0, 0.1^2)
    for zero-centred gains (scale 1 + g), 1 + N(0, 0.1^2) for plain gains."""
    if not cfg.prenorm:
        return None
    g = _rng(cfg.seed, "norm_gain", 0).standard_normal(cfg.d, dtype=np.float32) * 0.1
    if not cfg.norm_zero_centred:
        g = g + np.float32(1.0)
    return f32_to_bf16_bits(g) if cfg.dtype == "bf16" else g.astype(np.float32)


def make_sel_bias(cfg: MoEConfig) -> np.ndarray | None:
    if cfg.router != "sigmoid" or cfg.bias_std == 0.0:
        return None
    v = _rng(cfg.seed, "sel_bias", 0).standard_normal(size=cfg.E, dtype=np.float32)
    return (v * np.float32(cfg.bias_std)).astype(np.float32)


def zipf_ranks(cfg: MoEConfig) -> np.ndarray:
    """A seeded permutation of the popularity ranks 1..E over the routed experts."""
    return _rng(cfg.seed, "zipf_rank", 0).permutation(cfg.E).astype(np.int64) + 1


def stored_zipf_scale(cfg: MoEConfig) -> float:
    with open(_CALIB_FILE) as f:
        table = json.load(f)
    return float(table[cfg.name]["a"])


def make_logit_offset(cfg: MoEConfig, a: float | None = None) -> np.ndarray | None:
    """Per-expert logit offset o_e = -s * a * ln(rank_e) (the log of a Zipf(s) pmf without
    its normalizing constant), for the skewed workload; None otherwise.  ``a`` defaults
    to the calibrated value stored beside this module."""
    if cfg.zipf_s == 0.0:
        return None
    if a is None:
        a = stored_zipf_scale(cfg)
    r = zipf_ranks(cfg).astype(np.float64)
    return (-cfg.zipf_s * a * np.log(r)).astype(np.float32)


# ----------------------------------------------------------------------------- experts
EXPERT_TENSORS = ("w_gate", "w_up", "w_down")


def expert_shape(cfg: MoEConfig, tensor: str):
    return (cfg.d, cfg.I) if tensor == "w_down" else (cfg.I, cfg.d)


def make_expert(cfg: MoEConfig, tensor: str, e: int) -> np.ndarray:
    """One expert's matrix of ``tensor``: [I, d] for gate/up, [d, I] for down."""
    return _draw(_rng(cfg.seed, tensor, e), expert_shape(cfg, tensor), cfg.w_std, cfg.dtype)


def fill_expert_tensor(cfg: MoEConfig, tensor: str, out: np.ndarray | None = None,
                       experts=None, threads: int | None = None) -> np.ndarray:
    """Fill ``out`` [E + S, ...] with every (or the listed) expert's matrix, in parallel
    threads (NumPy's generators and ufuncs release the GIL)."""
    n = cfg.E + cfg.S
    if out is None:
        out = np.empty((n,) + expert_shape(cfg, tensor), storage_dtype(cfg))
    experts = range(n) if experts is None else experts

    def one(e):
        out[e] = make_expert(cfg, tensor, e)

    with ThreadPoolExecutor(threads or default_threads()) as ex:
        list(ex.map(one, experts))
    return out


# ----------------------------------------------------------------------------- MXFP4
# OCP Microscaling FP4 (the checkpoint format the pages name for Inkling's and K3's
# routed experts): 32 consecutive elements along K share one E8M0 scale byte s (scale
# 2^(s - 127)); each element is an E2M1 code (sign, 2 exponent bits, 1 mantissa bit), two
# codes per byte, element 2i in the low nibble.  Quantizing is input preparation here
# (the weights arrive quantized), not a step of the layer.
_E2M1_MAG = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], np.float64)
MX_BLOCK = 32


def quantize_mxfp4(w: np.ndarray):
    """float32 [..., K] -> (codes uint8 [..., K/2], scales uint8 [..., K/32]).  Per block,
    s = floor(log2(amax)) - 2 + 127 (amax / scale in [4, 8)); elements round to the
    nearest E2M1 magnitude, ties to the even code, saturating at 6."""
    w = np.asarray(w, np.float64)
    K = w.shape[-1]
    blocks = w.reshape(w.shape[:-1] + (K // MX_BLOCK, MX_BLOCK))
    amax = np.abs(blocks).max(axis=-1)
    with np.errstate(divide="ignore"):
        e = np.where(amax > 0, np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - 2, -127)
    s = np.clip(e + 127, 0, 254).astype(np.int64)
    a = np.abs(blocks) / np.ldexp(1.0, s - 127)[..., None]
    lo = np.clip(np.searchsorted(_E2M1_MAG, a, side="right") - 1, 0, 7)
    hi = np.minimum(lo + 1, 7)
    d_lo, d_hi = a - _E2M1_MAG[lo], _E2M1_MAG[hi] - a
    up = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0) & (hi != lo))
    mag = np.where(a >= 6.0, 7, np.where(up, hi, lo))
    code = (mag | np.where(blocks < 0, 8, 0)).astype(np.uint8)
    code = code.reshape(w.shape)
    packed = (code[..., 0::2] | (code[..., 1::2] << 4)).astype(np.uint8)
    return packed, s.astype(np.uint8)


def make_expert_mxfp4(cfg: MoEConfig, tensor: str, e: int):
    """Routed expert e's ``tensor`` in MXFP4: the same N(0, w_std^2) stream as the dense
    workloads, in float32, quantized."""
    return quantize_mxfp4(_draw(_rng(cfg.seed, tensor, e), expert_shape(cfg, tensor),
                                cfg.w_std, "f32"))


def fill_expert_mxfp4(cfg: MoEConfig, tensor: str, threads: int | None = None):
    """(codes [E, N, K/2], scales [E, N, K/32]) of every routed expert."""
    N, K = expert_shape(cfg, tensor)
    codes = np.empty((cfg.E, N, K // 2), np.uint8)
    scales = np.empty((cfg.E, N, K // MX_BLOCK), np.uint8)

    def one(e):
        codes[e], scales[e] = make_expert_mxfp4(cfg, tensor, e)

    with ThreadPoolExecutor(threads or default_threads()) as ex:
        list(ex.map(one, range(cfg.E)))
    return codes, scales


def make_inputs(cfg: MoEConfig, with_experts: bool = True, threads: int | None = None) -> dict:
    """All inputs of one workload as host arrays (bf16 as uint16 bits).  MXFP4 workloads
    hold the routed experts as ``wq_<tensor>`` (codes) and ``ws_<tensor>`` (scales) and
    only the S shared experts in ``w_<tensor>``."""
    inp = {
        "x": make_x(cfg),
        "w_router": make_w_router(cfg),
        "sel_bias": make_sel_bias(cfg),
        "logit_offset": make_logit_offset(cfg),
        "norm_gain": make_norm_gain(cfg),
    }
    if with_experts and cfg.weight_format == "mxfp4":
        for t in EXPERT_TENSORS:
            inp["wq_" + t[2:]], inp["ws_" + t[2:]] = fill_expert_mxfp4(cfg, t, threads)
            shared = np.empty((cfg.S,) + expert_shape(cfg, t), storage_dtype(cfg))
            for s_ in range(cfg.S):
                shared[s_] = make_expert(cfg, t, cfg.E + s_)
            inp[t] = shared
    elif with_experts:
        for t in EXPERT_TENSORS:
            inp[t] = fill_expert_tensor(cfg, t, threads=threads)
    return inp
