"""CPU oracle of the mixture-of-experts feed-forward layer.

TEST INFRASTRUCTURE ONLY.  This module defines what the layer computes, in float64 with
NumPy, as plainly as the pages state it.  Only the test suite, the smoke check and the
CPU-baseline leg of the benchmark may import it; the GPU library never calls it and shares
no code, header, table or helper with it.

What the layer computes (all citations are to the pages' component tables):

* Router.  A linear map of the token gives one score per expert (Qwen3.8-2.4T-A95B vs
  Inkling, component table, router row).  Two routers exist:
    - softmax top-k router: softmax over the routed experts, keep the top k, renormalize,
      no selection bias (same row, Qwen3.8 column; k = 10 of 512 per the Qwen3.8 2.4T
      A95B atlas page, raw config fields num_experts / num_experts_per_tok);
    - sigmoid router with shared-expert sink: sigmoid scores over the routed and the
      shared experts, top-k of the routed experts steered by a per-expert selection bias,
      weights normalized jointly over the k + S active experts then multiplied by their
      count (same row, Inkling column); a shared expert's weight is its own router
      score, taken into the same normalization as the routed experts' scores (Inkling vs
      Gemma 4 31B, component table, shared-expert row).
* Shared experts of the softmax router.  In the blueprint, one or two shared experts
  run on every token (Qwen3.5-397B-A17B vs Inkling, block diagram, shared-expert box),
  and the blueprint's shared expert carries no gate, unlike Inkling's router-weighted
  ones (Inkling vs Gemma 4 31B, component table, shared-expert row).  Qwen3.8 keeps one
  of intermediate size 2,048 (Qwen3.8 2.4T A95B atlas page, raw config
  shared_expert_intermediate_size).  Reading: its output is added with weight 1, outside
  the renormalized routed mixture, and it has no router row.
* Pre-norm (optional, the step before the layer).  Each block's branch input is the
  RMS-normalized residual stream ("Qwen3.5-397B-A17B vs Inkling" and "Qwen3.8-2.4T-A95B vs
  Inkling", residual-stream rows: pre-norm blocks; RMSNorm in the block diagrams).
  Qwen3.8's gains are zero-centred (same row), i.e. the scale is 1 + g, and its epsilon is
  1e-6 (Qwen3.8 2.4T A95B atlas page, raw config rms_norm_eps).  RMSNorm itself is the
  standard y = x / sqrt(mean(x^2) + eps) * gain.  bf16 layers take the normalized x
  rounded once to bf16 (nearest even) as their input.
* MXFP4 expert weights (optional).  The pages name block-scaled FP4 (MXFP4/NVFP4) for
  Inkling's routed experts (Qwen3.5-397B-A17B vs Inkling, block diagram, low-precision
  training box; Inkling vs Gemma 4 31B, shared-expert row: the shared experts stay BF16 in
  the FP4 checkpoint) but do not define the format; the OCP Microscaling definition is
  used: blocks of 32 elements along K, an E8M0 scale 2^(s - 127) per block, E2M1 elements
  (sign, 2 exponent bits with bias 1, 1 mantissa bit).  The layer then runs on the exact
  dequantized weights.
* Experts.  SwiGLU FFNs: E(x) = W_down (SiLU(W_gate x) * W_up x), SiLU(z) = z / (1 + e^-z)
  (Inkling vs Gemma 4 31B, routed-expert and shared-expert rows; Qwen3.8 2.4T A95B atlas
  page, key facts "Activation silu" and raw config hidden_act).
* Combine.  The weighted sum of the active experts' outputs is the branch output that is
  added back to the residual stream (Qwen3.5-397B-A17B vs Inkling, block diagram:
  router -> routed + shared experts -> residual add).

Readings where the pages leave a step open (each is listed in the design notes):
  - the selection bias is added to the sigmoid score (``bias_on_logits=False``); the
    other reading, bias added to the logit, is a flag;
  - the bias steers selection only; weights use the raw sigmoid scores;
  - shared experts' scores are the sigmoid of their own router rows (last S rows);
  - the softmax router's shared experts are ungated: weight exactly 1, no router row;
  - the "x8" constant is the active count k + S (``route_scale``);
  - ties in selection go to the lower expert index;
  - bf16 workloads ("bf16-flow" mode) round the SwiGLU intermediate h to bf16 once,
    round-to-nearest-even, as the bf16 input of the down projection; every sum is exact
    (float64) here;
  - a per-expert logit offset, when given, is added to the routed experts' logits before
    scoring (used only to skew the synthetic routing).

Inputs are the generator's exact values: bf16 tensors arrive as uint16 bit patterns and
are promoted exactly to float64; float32 tensors are promoted exactly.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


# ----------------------------------------------------------------------------- numbers
def promote(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 value of stored inputs: bf16 bit patterns (uint16) or float32.
    float64 arrays (values the oracle computed itself) pass through unchanged."""
    a = np.asarray(a)
    if a.dtype == np.float64:
        return a
    if dtype == "bf16":
        assert a.dtype == np.uint16, a.dtype
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    assert a.dtype == np.float32, a.dtype
    return a.astype(np.float64)


def round_to_bf16(v: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bf16 value (8 significant bits, ties to even,
    bf16's exponent range with gradual underflow).  Returns float64."""
    v = np.asarray(v, dtype=np.float64)
    _, e = np.frexp(v)                 # v = m * 2**e, 0.5 <= |m| < 1
    e = np.maximum(e, -125)            # below 2**-126 the spacing stays 2**-133
    return np.ldexp(np.rint(np.ldexp(v, 8 - e)), e - 8)


def sigmoid(z: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-z))


def silu(z: np.ndarray) -> np.ndarray:
    """SiLU(z) = z * sigmoid(z) (the pages' hidden_act "silu")."""
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def softmax(z: np.ndarray) -> np.ndarray:
    z = z - z.max(axis=-1, keepdims=True)
    ez = np.exp(z)
    return ez / ez.sum(axis=-1, keepdims=True)


# ----------------------------------------------------------------------------- pre-norm
def rmsnorm(x64: np.ndarray, gain64: np.ndarray, eps: float, gain_offset: float) -> np.ndarray:
    """RMSNorm of each row: x / sqrt(mean over the row of x^2 + eps) * (gain_offset + g).
    gain_offset is 1 for zero-centred gains (Qwen3.8), 0 for plain gains."""
    ms = np.mean(x64 * x64, axis=1, keepdims=True)
    return x64 / np.sqrt(ms + eps) * (gain_offset + gain64)


def prenorm_input(cfg, x, gain, eps: float, gain_offset: float, mode: str = "bf16_flow",
                  tokens=None) -> np.ndarray:
    """The layer's input for pre-norm blocks: RMSNorm of the raw hidden states x (all
    tokens, or the listed ones), as float64 values; bf16 layers in bf16-flow mode round
    it once to bf16, the precision in which the experts and the router read it."""
    xs = x if tokens is None else x[np.asarray(tokens)]
    y = rmsnorm(promote(xs, cfg.dtype), promote(gain, cfg.dtype), eps, gain_offset)
    if mode == "bf16_flow" and cfg.dtype == "bf16":
        y = round_to_bf16(y)
    return y


# ----------------------------------------------------------------------------- MXFP4
def e2m1_value(code: np.ndarray) -> np.ndarray:
    """E2M1 element value from its 4-bit code: sign bit 3, exponent bits 2..1 (bias 1),
    mantissa bit 0; exponent 0 is subnormal (0 or 0.5)."""
    code = np.asarray(code, np.int64)
    sign = np.where(code & 8, -1.0, 1.0)
    e = (code >> 1) & 3
    m = code & 1
    mag = np.where(e == 0, 0.5 * m, (1.0 + 0.5 * m) * np.ldexp(1.0, e - 1))
    return sign * mag


def e8m0_value(s: np.ndarray) -> np.ndarray:
    """E8M0 scale: 2^(s - 127); s = 255 is NaN."""
    s = np.asarray(s, np.int64)
    return np.where(s == 255, np.nan, np.ldexp(1.0, s - 127))


def dequant_mxfp4(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """[..., K/2] packed codes (element 2i in the low nibble) and [..., K/32] scales ->
    float64 [..., K]."""
    codes = np.asarray(codes, np.uint8)
    el = np.empty(codes.shape[:-1] + (2 * codes.shape[-1],), np.int64)
    el[..., 0::2] = codes & 0xF
    el[..., 1::2] = codes >> 4
    v = e2m1_value(el)
    K = v.shape[-1]
    v = v.reshape(v.shape[:-1] + (K // 32, 32)) * e8m0_value(scales)[..., None]
    return v.reshape(v.shape[:-2] + (K,))


def expert_weights(cfg, inputs: dict, e: int):
    """(W_gate, W_up, W_down) of expert e as float64: MXFP4 workloads keep the routed
    experts quantized (``wq_*`` codes, ``ws_*`` scales) and the shared experts, like every
    dense workload, in ``w_*`` (shared expert s at index s there)."""
    if getattr(cfg, "weight_format", "dense") == "mxfp4":
        if e < cfg.E:
            return tuple(dequant_mxfp4(inputs["wq_" + t][e], inputs["ws_" + t][e])
                         for t in ("gate", "up", "down"))
        e = e - cfg.E
    return tuple(promote(inputs["w_" + t][e], cfg.dtype) for t in ("gate", "up", "down"))


# ----------------------------------------------------------------------------- router
def router_logits(x64: np.ndarray, w_router64: np.ndarray, E: int,
                  logit_offset: np.ndarray | None = None) -> np.ndarray:
    """l = W_r x for every token (rows) and every expert, routed then shared (columns).
    No router bias exists on the pages.  ``logit_offset`` [E], if given, is added to the
    routed experts' logits."""
    l = x64 @ w_router64.T
    if logit_offset is not None:
        l[:, :E] += np.asarray(logit_offset, dtype=np.float64)
    return l


def top_k_descending(sel: np.ndarray, k: int):
    """The k largest entries of each row, in descending order; equal values keep the lower
    index first.  Also returns gap = k-th largest - (k+1)-th largest (inf when k = E)."""
    order = np.argsort(-sel, axis=1, kind="stable")
    srt = np.take_along_axis(sel, order, axis=1)
    if k < sel.shape[1]:
        gap = srt[:, k - 1] - srt[:, k]
    else:
        gap = np.full(sel.shape[0], np.inf)
    return order[:, :k].astype(np.int64), gap


@dataclass
class Routing:
    idx: np.ndarray      # [T, k] routed experts, descending selection score
    weights: np.ndarray  # [T, k + S] combine weights: routed (in idx order), then shared
    gap: np.ndarray      # [T] k-th minus (k+1)-th selection score
    sel: np.ndarray      # [T, E] selection scores (sigmoid: s + b; softmax: p)
    scores: np.ndarray   # [T, E + S] sigmoid scores s, or [T, E] softmax probabilities p
    logits: np.ndarray   # [T, E + S] (sigmoid) or [T, E] (softmax)
    counts: np.ndarray   # [E] tokens routed to each routed expert


def route_sigmoid_shared(logits: np.ndarray, E: int, S: int, k: int, route_scale: float,
                         sel_bias: np.ndarray | None, bias_on_logits: bool = False,
                         forced_idx: np.ndarray | None = None) -> Routing:
    """Sigmoid router with shared-expert sink (Qwen3.8-2.4T-A95B vs Inkling, component
    table, router row, Inkling column; Inkling vs Gemma 4 31B, shared-expert row).

    s_e = sigmoid(l_e) for all E + S experts.  The k routed experts with the largest
    selection score sel_e = s_e + b_e are kept (b steers selection only); the S shared
    experts are always active.  Over the active set A, w_j = route_scale * s_j / sum_A s.
    """
    s = sigmoid(logits)
    b = np.zeros(E) if sel_bias is None else np.asarray(sel_bias, dtype=np.float64)
    if bias_on_logits:
        sel = sigmoid(logits[:, :E] + b)
    else:
        sel = s[:, :E] + b
    idx, gap = top_k_descending(sel, k)
    if forced_idx is not None:
        idx = np.asarray(forced_idx, dtype=np.int64)
    s_active = np.concatenate([np.take_along_axis(s[:, :E], idx, axis=1), s[:, E:E + S]],
                              axis=1)
    w = route_scale * s_active / s_active.sum(axis=1, keepdims=True)
    counts = np.bincount(idx.ravel(), minlength=E)
    return Routing(idx, w, gap, sel, s, logits, counts)


def route_softmax_topk(logits: np.ndarray, E: int, k: int, S: int = 0,
                       forced_idx: np.ndarray | None = None) -> Routing:
    """Softmax top-k router (Qwen3.8-2.4T-A95B vs Inkling, component table, router row,
    Qwen3.8 column): p = softmax(l) over the E routed experts, keep the k largest,
    renormalize: w_j = p_j / sum_topk p.  No selection bias.  The S shared experts are
    ungated (the blueprint's shared expert; Inkling vs Gemma 4 31B, shared-expert row):
    weight 1 each, after the k routed weights."""
    p = softmax(logits[:, :E])
    idx, gap = top_k_descending(p, k)
    if forced_idx is not None:
        idx = np.asarray(forced_idx, dtype=np.int64)
    pa = np.take_along_axis(p, idx, axis=1)
    w = pa / pa.sum(axis=1, keepdims=True)
    w = np.concatenate([w, np.ones((w.shape[0], S))], axis=1)
    counts = np.bincount(idx.ravel(), minlength=E)
    return Routing(idx, w, gap, p, p, logits, counts)


def route(cfg, x, w_router, sel_bias=None, logit_offset=None, tokens=None,
          forced_idx=None) -> Routing:
    """Route the tokens of ``x`` (all, or the listed ``tokens``).  ``cfg`` supplies E, S,
    k, router, dtype, route_scale and bias_on_logits."""
    xs = x if tokens is None else x[np.asarray(tokens)]
    x64 = promote(xs, cfg.dtype)
    l = router_logits(x64, promote(w_router, cfg.dtype), cfg.E, logit_offset)
    if cfg.router == "sigmoid":
        return route_sigmoid_shared(l, cfg.E, cfg.S, cfg.k, cfg.route_scale, sel_bias,
                                    cfg.bias_on_logits, forced_idx)
    assert cfg.router == "softmax"
    return route_softmax_topk(l, cfg.E, cfg.k, cfg.S, forced_idx)


# ----------------------------------------------------------------------------- experts
def swiglu_expert(x64: np.ndarray, w_gate64: np.ndarray, w_up64: np.ndarray,
                  w_down64: np.ndarray, round_h_bf16: bool) -> np.ndarray:
    """One SwiGLU expert on rows x [n, d]: W_down (SiLU(W_gate x) * W_up x), with
    W_gate, W_up [I, d] and W_down [d, I] (Inkling vs Gemma 4 31B, routed-expert row).
    In bf16-flow mode h is rounded once to bf16 before the down projection."""
    g = x64 @ w_gate64.T
    u = x64 @ w_up64.T
    h = silu(g) * u
    if round_h_bf16:
        h = round_to_bf16(h)
    return h @ w_down64.T


@dataclass
class OracleOut:
    y: np.ndarray        # [n_tokens, d] branch output (plus residual if given)
    tokens: np.ndarray   # the token indices the rows of y belong to
    routing: Routing     # routing of those tokens


def moe_forward_prenorm(cfg, inputs: dict, gain, eps: float, gain_offset: float,
                        mode: str = "bf16_flow", tokens=None, forced_idx=None,
                        residual=None) -> OracleOut:
    """The pre-norm block's branch: the layer applied to RMSNorm(x) (``prenorm_input``);
    ``inputs["x"]`` holds the raw hidden states.  ``forced_idx`` and the residual act as
    in ``moe_forward``."""
    tok = np.arange(inputs["x"].shape[0]) if tokens is None else np.asarray(tokens)
    xn = np.zeros((inputs["x"].shape[0], cfg.d))
    xn[tok] = prenorm_input(cfg, inputs["x"], gain, eps, gain_offset, mode, tokens=tok)
    return moe_forward(cfg, dict(inputs, x=xn), mode=mode, tokens=tok,
                       forced_idx=forced_idx, residual=residual)


def moe_forward(cfg, inputs: dict, mode: str = "bf16_flow", tokens=None,
                forced_idx=None, residual=None) -> OracleOut:
    """The layer's output for all tokens, or the listed ``tokens``:
    y_t = sum over the active experts j of w_tj * E_j(x_t)   [+ residual_t].

    ``mode``: "bf16_flow" rounds h to bf16 (parity reference for bf16 workloads);
    "exact" rounds nothing.  float32 workloads are always exact.
    ``forced_idx`` [n, k] replaces the oracle's own routed selection (weights are then
    those of the forced set).
    ``inputs`` holds the generator's arrays: x, w_router, sel_bias, logit_offset,
    w_gate, w_up, w_down (and wq_* / ws_* for MXFP4 routed experts)."""
    x = inputs["x"]
    tok = np.arange(x.shape[0]) if tokens is None else np.asarray(tokens)
    r = route(cfg, x, inputs["w_router"], inputs.get("sel_bias"),
              inputs.get("logit_offset"), tokens=tok, forced_idx=forced_idx)
    round_h = (mode == "bf16_flow") and cfg.dtype == "bf16"
    x64 = promote(x[tok], cfg.dtype)
    n = len(tok)
    y = np.zeros((n, cfg.d))
    # Active set per token: routed (idx) then shared experts E .. E+S-1.
    active = np.concatenate([r.idx, np.broadcast_to(np.arange(cfg.E, cfg.E + cfg.S),
                                                    (n, cfg.S))], axis=1)
    for e in np.unique(active):
        rows, slots = np.nonzero(active == e)
        wg, wu, wd = expert_weights(cfg, inputs, int(e))
        out = swiglu_expert(x64[rows], wg, wu, wd, round_h)
        y[rows] += r.weights[rows, slots][:, None] * out
    if residual is not None:
        y = np.asarray(residual, dtype=np.float64)[tok] + y
    return OracleOut(y, tok, r)
