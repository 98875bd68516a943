"""Pins of the CPU oracle against facts that do not come from the oracle itself:
hand-derived closed forms, brute force, invariants the pages state, special cases that
reduce to a dense SwiGLU, and library routines.  CPU only."""
import itertools
import math

import numpy as np
import pytest

from moe_inputs import CONFIGS, MoEConfig, make_inputs
from moe_inputs.generate import f32_to_bf16_bits
from oracle import moe_oracle as O


def small_cfg(router="sigmoid", dtype="f32", T=24, d=16, E=8, S=2, I=12, k=3, seed=10,
              **kw):
    if router == "softmax":
        S = 0
    return MoEConfig(name=f"small_{router}_{dtype}", T=T, d=d, E=E, S=S, I=I, k=k,
                     router=router, dtype=dtype, x_std=1.0, w_std=0.3,
                     bias_std=0.1 if router == "sigmoid" else 0.0, zipf_s=0.0,
                     zipf_hot_share=0.0, seed=seed, **kw)


def shift_matrix(n, p):
    """P^p with P e_i = e_{(i+1) mod n}: column i has its 1 in row (i+p) mod n."""
    m = np.zeros((n, n))
    for i in range(n):
        m[(i + p) % n, i] = 1.0
    return m


def worked_inputs(E, S, logits, bias, experts):
    d = I = 4
    n = E + S
    w_router = np.zeros((n, d), np.float32)
    w_router[:, 0] = np.asarray(logits, np.float32)
    x = np.zeros((1, d), np.float32)
    x[0, 0] = 1.0
    wg = np.zeros((n, I, d), np.float32)
    wu = np.zeros((n, I, d), np.float32)
    wd = np.zeros((n, d, I), np.float32)
    for j, (a, c, m, p) in enumerate(experts):
        wg[j] = a * np.eye(4)
        wu[j] = c * np.eye(4)
        wd[j] = m * shift_matrix(4, p)
    return {"x": x, "w_router": w_router,
            "sel_bias": None if bias is None else np.asarray(bias, np.float32),
            "logit_offset": None, "w_gate": wg, "w_up": wu, "w_down": wd}


# ---------------------------------------------------------------- worked examples (golden)
def test_worked_example_sigmoid_shared():
    """tests/golden/worked_examples.md, Example A."""
    ln3, ln7 = math.log(3), math.log(7)
    cfg = MoEConfig(name="wA", T=1, d=4, E=4, S=1, I=4, k=2, router="sigmoid", dtype="f32",
                    x_std=1, w_std=1, bias_std=0.1, zipf_s=0, zipf_hot_share=0, seed=0)
    experts = [(-ln3, 1, 1, 2), (ln3, 2, 1, 1), (1, 1, 1, 3), (1, 1, 1, 3), (ln7, 1, 2, 0)]
    inp = worked_inputs(4, 1, [ln3, 0, -ln3, ln7, 0], [0, 0.5, 0, -0.2], experts)
    out = O.moe_forward(cfg, inp, mode="exact")
    assert out.routing.idx.tolist() == [[1, 0]]
    np.testing.assert_allclose(out.routing.gap, [0.075], rtol=1e-6)
    np.testing.assert_allclose(out.routing.weights, [[6 / 7, 9 / 7, 6 / 7]], rtol=1e-6)
    np.testing.assert_allclose(out.y, [[1.5 * ln7, 9 / 7 * ln3, -9 / 28 * ln3, 0]],
                               rtol=1e-6, atol=1e-7)
    # The other reading of the bias (on the logit) selects differently: this fixture
    # tells the two apart.
    out2 = O.moe_forward(cfg.with_(bias_on_logits=True), inp, mode="exact")
    assert out2.routing.idx.tolist() == [[3, 0]]


def test_worked_example_softmax_topk():
    """tests/golden/worked_examples.md, Example B."""
    ln3, ln7 = math.log(3), math.log(7)
    cfg = MoEConfig(name="wB", T=1, d=4, E=4, S=0, I=4, k=2, router="softmax", dtype="f32",
                    x_std=1, w_std=1, bias_std=0, zipf_s=0, zipf_hot_share=0, seed=0)
    experts = [(ln3, 1, 1, 1), (1, 1, 1, 3), (1, 1, 1, 3), (ln7, 2, 1, 2)]
    inp = worked_inputs(4, 0, [math.log(4), math.log(2), 0, ln3], None, experts)
    out = O.moe_forward(cfg, inp, mode="exact")
    assert out.routing.idx.tolist() == [[0, 3]]
    np.testing.assert_allclose(out.routing.gap, [0.1], rtol=1e-6)
    np.testing.assert_allclose(out.routing.weights, [[4 / 7, 3 / 7]], rtol=1e-6)
    np.testing.assert_allclose(out.y, [[0, 3 / 7 * ln3, 0.75 * ln7, 0]], rtol=1e-6,
                               atol=1e-7)


def test_worked_example_softmax_ungated_shared():
    """tests/golden/worked_examples.md, Example C."""
    ln3, ln7 = math.log(3), math.log(7)
    cfg = MoEConfig(name="wC", T=1, d=4, E=3, S=1, I=4, k=2, router="softmax", dtype="f32",
                    x_std=1, w_std=1, bias_std=0, zipf_s=0, zipf_hot_share=0, seed=0)
    experts = [(ln3, 1, 1, 1), (1, 1, 1, 3), (ln7, 2, 1, 2), (-ln3, 1, 2, 0)]
    inp = worked_inputs(3, 1, [ln3, 0, math.log(2), 0], None, experts)
    inp["w_router"] = inp["w_router"][:3]          # the shared expert has no router row
    out = O.moe_forward(cfg, inp, mode="exact")
    assert out.routing.idx.tolist() == [[0, 2]]
    np.testing.assert_allclose(out.routing.gap, [1 / 6], rtol=1e-6)
    np.testing.assert_allclose(out.routing.weights, [[3 / 5, 2 / 5, 1]], rtol=1e-6)
    np.testing.assert_allclose(out.y, [[-0.5 * ln3, 0.45 * ln3, 0.7 * ln7, 0]], rtol=1e-6,
                               atol=1e-7)


# ---------------------------------------------------------------- numbers
def test_promote_bf16_bit_patterns():
    bits = np.array([0x3F80, 0xC000, 0x0001, 0x7F7F, 0x0000, 0x8000, 0x3F81], np.uint16)
    want = [1.0, -2.0, 2.0 ** -133, (2 - 2 ** -7) * 2.0 ** 127, 0.0, -0.0, 1 + 2 ** -7]
    assert O.promote(bits, "bf16").tolist() == want


def test_round_to_bf16_ties_and_subnormals():
    v = np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8 + 2 ** -30), 2 ** -134,
                  3 * 2 ** -134, 2 ** -126 * (1 + 2 ** -8)])
    want = [1.0, 1 + 2 ** -6, -(1 + 2 ** -7), 0.0, 2 * 2 ** -133, 2 ** -126]
    assert O.round_to_bf16(v).tolist() == want


def test_round_to_bf16_matches_torch_on_float32():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(0)
    v = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 3,
                        (rng.standard_normal(20000) * 1e-39).astype(np.float32),
                        rng.integers(0, 2 ** 32, 20000, dtype=np.uint64).astype(np.uint32)
                        .view(np.float32)])
    v = v[np.isfinite(v) & (np.abs(v) < 3e38)]
    mine = O.round_to_bf16(v.astype(np.float64))
    ref = torch.from_numpy(v).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(mine, ref)


# ---------------------------------------------------------------- pre-norm
def test_rmsnorm_closed_form():
    """x = (3, 4, 0, 0): mean of squares 25/4, rms 5/2, so x / rms = (1.2, 1.6, 0, 0);
    zero-centred gains g scale by 1 + g, plain gains by g."""
    x = np.array([[3.0, 4.0, 0.0, 0.0]])
    g = np.array([0.5, -0.25, 2.0, 1.0])
    np.testing.assert_allclose(O.rmsnorm(x, g, 0.0, 0.0), [[0.6, -0.4, 0, 0]], rtol=1e-15)
    np.testing.assert_allclose(O.rmsnorm(x, g, 0.0, 1.0), [[1.8, 1.2, 0, 0]], rtol=1e-15)
    # eps enters under the root: mean 25/4 + 3/4 = 7, rms sqrt(7)
    np.testing.assert_allclose(O.rmsnorm(x, np.ones(4), 0.75, 0.0),
                               [[3 / math.sqrt(7), 4 / math.sqrt(7), 0, 0]], rtol=1e-15)


def test_rmsnorm_matches_torch():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(3)
    x = rng.standard_normal((64, 384)) * 3.0
    g = rng.standard_normal(384) * 0.1
    ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (384,), torch.from_numpy(1 + g),
                                       eps=1e-6).numpy()
    np.testing.assert_allclose(O.rmsnorm(x, g, 1e-6, 1.0), ref, rtol=1e-13, atol=1e-13)


def test_rmsnorm_scale_invariance_and_prenorm_rounding():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((16, 64))
    g = 1 + 0.1 * rng.standard_normal(64)
    np.testing.assert_allclose(O.rmsnorm(1e3 * x, g, 0.0, 0.0), O.rmsnorm(x, g, 0.0, 0.0),
                               rtol=1e-13)
    cfg = small_cfg("sigmoid", dtype="bf16", T=16, d=64).with_(prenorm=True)
    inp = make_inputs(cfg, with_experts=False)
    xn = O.prenorm_input(cfg, inp["x"], inp["norm_gain"], cfg.norm_eps, 0.0)
    exact = O.prenorm_input(cfg, inp["x"], inp["norm_gain"], cfg.norm_eps, 0.0, mode="exact")
    assert (O.round_to_bf16(exact) == xn).all()
    assert 0 < np.abs(xn - exact).max() <= 2.0 ** -8 * np.abs(exact).max()


# ---------------------------------------------------------------- MXFP4 weights
def test_e2m1_code_table():
    """The 16 E2M1 codes: sign, 2 exponent bits (bias 1), 1 mantissa bit; exponent 0 is
    subnormal.  Magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6 (the OCP MX element table)."""
    want = [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    got = O.e2m1_value(np.arange(16))
    assert got[:8].tolist() == want
    assert got[8:].tolist() == [-v for v in want]
    assert math.copysign(1.0, got[8]) == -1.0          # code 8 is -0


def test_e8m0_scale():
    v = O.e8m0_value(np.array([0, 1, 126, 127, 128, 254, 255]))
    assert v[:6].tolist() == [2.0 ** -127, 2.0 ** -126, 0.5, 1.0, 2.0, 2.0 ** 127]
    assert np.isnan(v[6])


def test_dequant_mxfp4_hand_example():
    """Byte 0x21 holds element 0 = code 1 (0.5) in its low nibble and element 1 = code 2
    (1.0) in its high nibble; byte 0xF8 holds -0 and -6.  Scale byte 128 doubles them."""
    codes = np.zeros((1, 16), np.uint8)
    codes[0, :2] = [0x21, 0xF8]
    codes[0, 2] = 0x7F                                   # -6, then +6
    v = O.dequant_mxfp4(codes, np.array([[128]], np.uint8))
    assert v[0, :6].tolist() == [1.0, 2.0, -0.0, -12.0, -12.0, 12.0]
    assert (v[0, 6:] == 0).all()
    # A second block has its own scale.
    codes2 = np.zeros((1, 32), np.uint8)
    codes2[0, 16] = 0x33                                 # elements 32, 33 = 1.5 each
    v2 = O.dequant_mxfp4(codes2, np.array([[127, 125]], np.uint8))
    assert v2[0, 32:34].tolist() == [0.375, 0.375] and v2[0, :32].sum() == 0


def test_mxfp4_round_trip_and_error_bound():
    """The generator's quantizer (written separately) against the oracle's decoder:
    grid values times a block scale come back exactly, and random weights land within
    the format's step (at most 2 scale units, past the largest element 6)."""
    from moe_inputs import quantize_mxfp4
    rng = np.random.default_rng(9)
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], np.float32)
    exact = (rng.choice(grid, (8, 64)) * rng.choice([-1, 1], (8, 64))).astype(np.float32)
    exact[:, 0] = 6.0                                    # pins each block's scale to 1
    exact[:, 32] = -6.0
    c, sc = quantize_mxfp4(exact)
    assert (sc == 127).all()
    np.testing.assert_array_equal(O.dequant_mxfp4(c, sc), exact)
    w = (rng.standard_normal((16, 256)) * 0.02).astype(np.float32)
    c, sc = quantize_mxfp4(w)
    err = np.abs(O.dequant_mxfp4(c, sc) - w).reshape(16, 8, 32)
    scale = O.e8m0_value(sc)[..., None]
    assert (err <= 2 * scale).all() and (err <= 0.5 * scale).mean() > 0.5


def test_mxfp4_workload_uses_dequantized_routed_and_bf16_shared_weights():
    cfg = small_cfg("sigmoid", dtype="bf16", T=12, d=64, E=6, S=1, I=32, k=2,
                    seed=15).with_(weight_format="mxfp4")
    inp = make_inputs(cfg)
    assert inp["wq_gate"].shape == (6, 32, 32) and inp["ws_down"].shape == (6, 64, 1)
    assert inp["w_gate"].shape == (1, 32, 64)
    out = O.moe_forward(cfg, inp, mode="exact")
    # The same layer with the dequantized weights stored densely (float64 passthrough).
    dense = dict(inp)
    for t in ("gate", "up", "down"):
        deq = O.dequant_mxfp4(inp["wq_" + t], inp["ws_" + t])
        dense["w_" + t] = np.concatenate([deq, O.promote(inp["w_" + t], "bf16")])
    ref = O.moe_forward(cfg.with_(weight_format="dense"), dense, mode="exact")
    np.testing.assert_allclose(out.y, ref.y, rtol=1e-13, atol=1e-15)


# ---------------------------------------------------------------- router
def test_topk_brute_force_subsets():
    rng = np.random.default_rng(1)
    for E, k in [(5, 1), (6, 2), (9, 3), (12, 4), (10, 10)]:
        sel = rng.standard_normal((40, E))
        idx, gap = O.top_k_descending(sel, k)
        for t in range(sel.shape[0]):
            best = max(itertools.combinations(range(E), k),
                       key=lambda c: sum(sel[t, list(c)]))
            assert set(idx[t]) == set(best)
            vals = sel[t, idx[t]]
            assert np.all(np.diff(vals) < 0)
            rest = np.setdiff1d(np.arange(E), idx[t])
            if k < E:
                assert gap[t] == pytest.approx(vals[-1] - sel[t, rest].max())


def test_tie_rule_zero_router_softmax():
    """W_r = 0: every softmax probability is 1/E; ties go to the lower index, so every
    token keeps experts 0..k-1 with weight 1/k."""
    cfg = small_cfg("softmax", E=9, k=4)
    inp = make_inputs(cfg)
    inp["w_router"] = np.zeros_like(inp["w_router"])
    r = O.route(cfg, inp["x"], inp["w_router"])
    assert (r.idx == np.arange(4)).all()
    np.testing.assert_allclose(r.weights, 0.25, rtol=0, atol=1e-15)
    assert (r.gap == 0).all()


@pytest.mark.parametrize("router", ["sigmoid", "softmax"])
def test_weights_sum_and_sign(router):
    cfg = small_cfg(router, T=200, E=16, k=4)
    inp = make_inputs(cfg)
    r = O.route(cfg, inp["x"], inp["w_router"], inp["sel_bias"])
    want = cfg.k + cfg.S if router == "sigmoid" else 1.0
    np.testing.assert_allclose(r.weights.sum(1), want, rtol=0, atol=1e-12)
    assert (r.weights > 0).all()
    assert r.counts.sum() == cfg.T * cfg.k
    assert all(len(set(row)) == cfg.k for row in r.idx.tolist())


def test_softmax_renormalized_equals_softmax_over_topk_logits():
    """Renormalized top-k softmax weights equal exp(l_j)/sum over the top-k of exp(l_i):
    the full E-way denominator cancels."""
    cfg = small_cfg("softmax", T=100, E=32, k=6)
    inp = make_inputs(cfg)
    r = O.route(cfg, inp["x"], inp["w_router"])
    la = np.take_along_axis(r.logits, r.idx, 1)
    closed = np.exp(la - la.max(1, keepdims=True))
    closed /= closed.sum(1, keepdims=True)
    np.testing.assert_allclose(r.weights, closed, rtol=1e-12)
    # top-k of probabilities == top-k of logits (monotone)
    assert (np.argsort(-r.logits, 1, kind="stable")[:, :cfg.k] == r.idx).all()


def test_sigmoid_weights_use_raw_scores_and_bias_only_selects():
    cfg = small_cfg("sigmoid", T=64, E=10, S=2, k=3)
    inp = make_inputs(cfg)
    r = O.route(cfg, inp["x"], inp["w_router"], inp["sel_bias"])
    s = 1 / (1 + np.exp(-r.logits))
    sa = np.concatenate([np.take_along_axis(s[:, :10], r.idx, 1), s[:, 10:]], 1)
    np.testing.assert_allclose(r.weights, 5 * sa / sa.sum(1, keepdims=True), rtol=1e-12)
    np.testing.assert_allclose(r.sel, s[:, :10] + inp["sel_bias"].astype(np.float64),
                               rtol=0, atol=1e-15)


# ---------------------------------------------------------------- experts and combine
def dense_swiglu(x, wg, wu, wd):
    g = x @ wg.T
    u = x @ wu.T
    return (g / (1 + np.exp(-g)) * u) @ wd.T


@pytest.mark.parametrize("router", ["sigmoid", "softmax"])
def test_identical_experts_give_scaled_dense_swiglu(router):
    """All experts equal => y = (sum of weights) * SwiGLU(x): 8x for the Inkling-style
    sigmoid router here k + S, 1x for softmax renormalization."""
    cfg = small_cfg(router, T=50, E=8, k=3)
    inp = make_inputs(cfg)
    for t in ("w_gate", "w_up", "w_down"):
        inp[t][:] = inp[t][0]
    out = O.moe_forward(cfg, inp, mode="exact")
    x = inp["x"].astype(np.float64)
    ref = dense_swiglu(x, inp["w_gate"][0].astype(np.float64),
                       inp["w_up"][0].astype(np.float64), inp["w_down"][0].astype(np.float64))
    np.testing.assert_allclose(out.y, cfg.route_scale * ref, rtol=1e-10, atol=1e-13)


def test_zero_router_sigmoid_is_dense_swiglu_of_stacked_experts():
    """W_r = 0 with the sigmoid router: s = 1/2 for every expert, so every token keeps the
    k experts with the largest bias, all weights are 1, and the layer is one dense SwiGLU
    of width (k + S) I built from the active experts (Inkling: 8 x 3,072 = 24,576, the
    width of its dense blocks, Inkling vs Gemma 4 31B, routed-expert row)."""
    cfg = small_cfg("sigmoid", T=40, E=12, S=2, k=6)
    inp = make_inputs(cfg)
    inp["w_router"] = np.zeros_like(inp["w_router"])
    out = O.moe_forward(cfg, inp, mode="exact")
    b = inp["sel_bias"]
    top = list(np.argsort(-b.astype(np.float64), kind="stable")[:6])
    assert (out.routing.idx == np.array(top)).all()
    np.testing.assert_allclose(out.routing.weights, 1.0, rtol=0, atol=1e-15)
    act = top + [12, 13]
    wg = np.concatenate([inp["w_gate"][j] for j in act]).astype(np.float64)
    wu = np.concatenate([inp["w_up"][j] for j in act]).astype(np.float64)
    wd = np.concatenate([inp["w_down"][j] for j in act], axis=1).astype(np.float64)
    assert wg.shape == (8 * cfg.I, cfg.d)
    ref = dense_swiglu(inp["x"].astype(np.float64), wg, wu, wd)
    np.testing.assert_allclose(out.y, ref, rtol=1e-10, atol=1e-13)


def test_silu_special_values():
    z = np.array([0.0, math.log(3), -math.log(3), math.log(7), 40.0, -40.0])
    want = [0.0, 0.75 * math.log(3), -0.25 * math.log(3), 0.875 * math.log(7), 40.0,
            -40.0 / (1 + math.exp(40))]
    np.testing.assert_allclose(O.silu(z), want, rtol=1e-14, atol=0)


@pytest.mark.parametrize("router", ["sigmoid", "softmax"])
def test_linearity_zero_input_and_token_permutation(router):
    cfg = small_cfg(router, T=30, E=8, k=2)
    inp = make_inputs(cfg)
    y = O.moe_forward(cfg, inp, mode="exact").y
    scaled = dict(inp, w_down=(inp["w_down"] * np.float32(0.5)))
    np.testing.assert_allclose(O.moe_forward(cfg, scaled, mode="exact").y, 0.5 * y,
                               rtol=1e-12, atol=1e-15)
    zero = dict(inp, x=np.zeros_like(inp["x"]))
    assert np.all(O.moe_forward(cfg, zero, mode="exact").y == 0)
    perm = np.random.default_rng(3).permutation(cfg.T)
    pinp = dict(inp, x=inp["x"][perm])
    pout = O.moe_forward(cfg, pinp, mode="exact")
    np.testing.assert_allclose(pout.y, y[perm], rtol=1e-12, atol=1e-15)
    base = O.route(cfg, inp["x"], inp["w_router"], inp["sel_bias"])
    assert (pout.routing.idx == base.idx[perm]).all()


def per_token_reference(cfg, inp, round_h):
    """A pure-Python loop over tokens and experts, written straight from the definition;
    independent of the oracle's vectorized gather/scatter."""
    def f(a):
        return O.promote(a, cfg.dtype)
    x, wr = f(inp["x"]), f(inp["w_router"])
    b = inp["sel_bias"]
    E, S, k = cfg.E, cfg.S, cfg.k
    ys, idxs, ws = [], [], []
    for t in range(cfg.T):
        logits = [sum(x[t, c] * wr[e, c] for c in range(cfg.d))
                  for e in range(cfg.router_rows)]
        if cfg.router == "sigmoid":
            s = [1 / (1 + math.exp(-v)) for v in logits]
            sel = [s[e] + float(b[e]) for e in range(E)]
            chosen = sorted(range(E), key=lambda e: (-sel[e], e))[:k]
            act = chosen + list(range(E, E + S))
            tot = sum(s[e] for e in act)
            w = [cfg.route_scale * s[e] / tot for e in act]
        else:
            m = max(logits)
            ex = [math.exp(v - m) for v in logits]
            z = sum(ex)
            p = [v / z for v in ex]
            chosen = sorted(range(E), key=lambda e: (-p[e], e))[:k]
            tot = sum(p[e] for e in chosen)
            # ungated shared experts: weight 1 each, outside the renormalization
            act = chosen + list(range(E, E + S))
            w = [p[e] / tot for e in chosen] + [1.0] * S
        y = [0.0] * cfg.d
        for wj, e in zip(w, act):
            wg, wu, wd = f(inp["w_gate"][e]), f(inp["w_up"][e]), f(inp["w_down"][e])
            h = []
            for i in range(cfg.I):
                g = sum(wg[i, c] * x[t, c] for c in range(cfg.d))
                u = sum(wu[i, c] * x[t, c] for c in range(cfg.d))
                hv = g / (1 + math.exp(-g)) * u
                h.append(float(O.round_to_bf16(np.array(hv))) if round_h else hv)
            for c in range(cfg.d):
                y[c] += wj * sum(wd[c, i] * h[i] for i in range(cfg.I))
        ys.append(y)
        idxs.append(chosen)
        ws.append(w)
    return np.array(ys), np.array(idxs), np.array(ws)


@pytest.mark.parametrize("router,dtype", [("sigmoid", "f32"), ("softmax", "f32"),
                                          ("sigmoid", "bf16"), ("softmax", "bf16")])
def test_oracle_matches_per_token_loop(router, dtype):
    cfg = small_cfg(router, dtype=dtype, T=6, d=8, E=6, S=2, I=5, k=2, seed=11)
    inp = make_inputs(cfg)
    mode = "bf16_flow" if dtype == "bf16" else "exact"
    out = O.moe_forward(cfg, inp, mode=mode)
    y, idx, w = per_token_reference(cfg, inp, round_h=(dtype == "bf16"))
    assert (out.routing.idx == idx).all()
    np.testing.assert_allclose(out.routing.weights, w, rtol=1e-12)
    np.testing.assert_allclose(out.y, y, rtol=1e-9, atol=1e-12)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_oracle_matches_per_token_loop_softmax_shared(dtype):
    cfg = MoEConfig(name="soft_shared", T=6, d=8, E=6, S=2, I=5, k=2, router="softmax",
                    dtype=dtype, x_std=1.0, w_std=0.3, bias_std=0.0, zipf_s=0.0,
                    zipf_hot_share=0.0, seed=13)
    inp = make_inputs(cfg)
    assert inp["w_router"].shape == (cfg.E, cfg.d)
    mode = "bf16_flow" if dtype == "bf16" else "exact"
    out = O.moe_forward(cfg, inp, mode=mode)
    y, idx, w = per_token_reference(cfg, inp, round_h=(dtype == "bf16"))
    assert (out.routing.idx == idx).all()
    np.testing.assert_allclose(out.routing.weights, w, rtol=1e-12)
    np.testing.assert_allclose(out.y, y, rtol=1e-9, atol=1e-12)


def test_ungated_shared_expert_adds_its_dense_output():
    """With the shared experts the softmax layer's output is the routed-only output (the
    same routing) plus, for every token, the plain sum of the shared experts' SwiGLU
    outputs: nothing renormalizes them and no score scales them."""
    cfg = MoEConfig(name="soft_shared2", T=16, d=16, E=8, S=2, I=12, k=3, router="softmax",
                    dtype="f32", x_std=1.0, w_std=0.3, bias_std=0.0, zipf_s=0.0,
                    zipf_hot_share=0.0, seed=14)
    inp = make_inputs(cfg)
    with_shared = O.moe_forward(cfg, inp, mode="exact")
    routed_only = O.moe_forward(cfg.with_(S=0), inp, mode="exact")
    assert (with_shared.routing.idx == routed_only.routing.idx).all()
    np.testing.assert_allclose(with_shared.routing.weights[:, :cfg.k],
                               routed_only.routing.weights, rtol=1e-15)
    x = inp["x"].astype(np.float64)
    dense = np.zeros_like(with_shared.y)
    for s in range(cfg.S):
        e = cfg.E + s
        g = x @ inp["w_gate"][e].astype(np.float64).T
        u = x @ inp["w_up"][e].astype(np.float64).T
        dense += (g * u / (1 + np.exp(-g))) @ inp["w_down"][e].astype(np.float64).T
    np.testing.assert_allclose(with_shared.y - routed_only.y, dense, rtol=1e-9, atol=1e-12)


def nearest_bf16_bits(v: float) -> int:
    """Bit pattern of the bf16 value nearest to v, ties to the even pattern: the bf16
    values around v's float32 pattern truncated to its upper 16 bits are compared with v
    in exact rational arithmetic (no frexp / rint)."""
    from fractions import Fraction
    import struct

    def val(bits):
        return struct.unpack("<f", struct.pack("<I", (bits & 0xFFFF) << 16))[0]
    hi16 = struct.unpack("<I", struct.pack("<f", v))[0] >> 16
    sign = hi16 & 0x8000
    mag = hi16 & 0x7FFF
    cands = [sign | m for m in (mag - 1, mag, mag + 1) if 0 <= m < 0x7F80]
    fv = Fraction(v)
    return min(cands, key=lambda b: (abs(Fraction(val(b)) - fv), b & 1))


@pytest.mark.parametrize("router,zc", [("sigmoid", False), ("softmax", True)])
def test_prenorm_layer_is_the_layer_on_the_rounded_normalized_input(router, zc):
    """moe_forward_prenorm: each token normalized by its RMS (plain Python sums), scaled
    by its gain (1 + g for zero-centred gains), rounded once to the nearest bf16, and then
    routed and run through the experts by the pure-Python per-token loop."""
    cfg = small_cfg(router, dtype="bf16", T=6, d=8, E=6, S=2, I=5, k=2, seed=16).with_(
        prenorm=True, norm_zero_centred=zc)
    if router == "softmax":
        cfg = cfg.with_(S=1)
    inp = make_inputs(cfg)
    off = 1.0 if zc else 0.0
    x = O.promote(inp["x"], "bf16")
    g = O.promote(inp["norm_gain"], "bf16")
    xn_bits = np.zeros(x.shape, np.uint16)
    for t in range(cfg.T):
        rms = math.sqrt(sum(v * v for v in x[t]) / cfg.d + cfg.norm_eps)
        for c in range(cfg.d):
            xn_bits[t, c] = nearest_bf16_bits(x[t, c] / rms * (off + g[c]))
    y, idx, w = per_token_reference(cfg, dict(inp, x=xn_bits), round_h=True)
    out = O.moe_forward_prenorm(cfg, inp, inp["norm_gain"], cfg.norm_eps, off,
                                mode="bf16_flow")
    assert (out.routing.idx == idx).all()
    np.testing.assert_allclose(out.routing.weights, w, rtol=1e-12)
    np.testing.assert_allclose(out.y, y, rtol=1e-9, atol=1e-12)
    # The same set in another order (forced routing) gives the same output.
    forced = O.moe_forward_prenorm(cfg, inp, inp["norm_gain"], cfg.norm_eps, off,
                                   mode="bf16_flow", forced_idx=idx[:, ::-1].copy())
    np.testing.assert_allclose(forced.y, y, rtol=1e-9, atol=1e-12)


def test_nearest_bf16_bits_against_torch():
    """The bracketing rounding above agrees with torch's float32 -> bf16 conversion on
    float32 inputs (single rounding there), ties and subnormals included."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(8)
    v = np.concatenate([rng.standard_normal(300).astype(np.float32),
                        np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, -(1 + 2.0 ** -8),
                                  2.0 ** -130, 3 * 2.0 ** -134], np.float32)])
    want = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([nearest_bf16_bits(float(a)) for a in v], np.uint16)
    np.testing.assert_array_equal(got, want)


def test_forced_routing_takes_the_forced_set_and_its_own_weights():
    """Forcing a different routed set: the output is the per-token definition on that set,
    weighted by the oracle's own raw scores of the forced experts, normalized over it."""
    cfg = small_cfg("sigmoid", T=8, E=8, S=2, k=2, seed=17)
    inp = make_inputs(cfg)
    r = O.route(cfg, inp["x"], inp["w_router"], inp["sel_bias"])
    # the 3rd-ranked expert in place of the 2nd
    order = np.argsort(-r.sel, axis=1, kind="stable")
    forced = np.stack([order[:, 0], order[:, 2]], 1)
    out = O.moe_forward(cfg, inp, mode="exact", forced_idx=forced)
    x = inp["x"].astype(np.float64)
    for t in range(cfg.T):
        act = list(forced[t]) + list(range(cfg.E, cfg.E + cfg.S))
        s = [r.scores[t, e] for e in act]
        want = np.zeros(cfg.d)
        for e, se in zip(act, s):
            gg = inp["w_gate"][e].astype(np.float64) @ x[t]
            uu = inp["w_up"][e].astype(np.float64) @ x[t]
            want += cfg.route_scale * se / sum(s) * (
                inp["w_down"][e].astype(np.float64) @ (gg * uu / (1 + np.exp(-gg))))
        np.testing.assert_allclose(out.y[t], want, rtol=1e-9, atol=1e-12)


def test_bf16_flow_differs_from_exact_at_the_single_rounding_point():
    """bf16-flow rounds only h; against the exact result the difference is the size of
    one bf16 rounding of h (relative 2^-9), far from zero and far below 1e-2."""
    cfg = small_cfg("sigmoid", dtype="bf16", T=64, d=256, E=8, S=2, I=256, k=2, seed=12)
    cfg = cfg.with_(w_std=0.02)
    inp = make_inputs(cfg)
    a = O.moe_forward(cfg, inp, mode="bf16_flow").y
    b = O.moe_forward(cfg, inp, mode="exact").y
    rms = np.sqrt(np.mean(b ** 2))
    rel = np.mean(np.abs(a - b)) / rms
    assert 1e-4 < rel < 5e-3


def test_forced_routing_reweights_the_forced_set():
    cfg = small_cfg("sigmoid", T=20, E=8, S=2, k=2)
    inp = make_inputs(cfg)
    r = O.route(cfg, inp["x"], inp["w_router"], inp["sel_bias"])
    forced = r.idx[:, ::-1].copy()          # same sets, reversed order
    out = O.moe_forward(cfg, inp, mode="exact", forced_idx=forced)
    base = O.moe_forward(cfg, inp, mode="exact")
    np.testing.assert_allclose(out.y, base.y, rtol=1e-12, atol=1e-15)


def test_residual_is_added():
    cfg = small_cfg("softmax", T=10, E=6, k=2)
    inp = make_inputs(cfg)
    res = np.random.default_rng(0).standard_normal((cfg.T, cfg.d)).astype(np.float32)
    a = O.moe_forward(cfg, inp, mode="exact", residual=res).y
    b = O.moe_forward(cfg, inp, mode="exact").y
    np.testing.assert_allclose(a - b, res, rtol=1e-12, atol=1e-12)


def test_generator_bf16_rounding_matches_torch():
    torch = pytest.importorskip("torch")
    v = np.random.default_rng(5).standard_normal(50000).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert (f32_to_bf16_bits(v) == ref).all()


def test_zipf_calibration_reproduces_hot_share():
    """The stored Zipf scale gives the skewed workload its 30% +- 0.5% hot-8 share under
    the oracle's routing."""
    cfg = CONFIGS["inkling_skewed"]
    inp = make_inputs(cfg, with_experts=False)
    r = O.route(cfg, inp["x"], inp["w_router"], inp["sel_bias"], inp["logit_offset"])
    from moe_inputs.generate import zipf_ranks
    hot = np.nonzero(zipf_ranks(cfg) <= 8)[0]
    share = r.counts[hot].sum() / (cfg.T * cfg.k)
    assert abs(share - 0.30) <= 0.005


def test_tie_rule_duplicate_router_rows():
    """Experts 3 and 7 share one router row, so their scores tie for every token; whenever
    exactly one of them is kept it must be the lower index, 3."""
    cfg = small_cfg("sigmoid", T=400, E=40, S=2, k=6).with_(bias_std=0.0)
    inp = make_inputs(cfg)
    inp["w_router"][7] = inp["w_router"][3]
    r = O.route(cfg, inp["x"], inp["w_router"], None)
    has3 = (r.idx == 3).any(1)
    has7 = (r.idx == 7).any(1)
    assert has3.sum() > 10
    assert not (has7 & ~has3).any()
    both = has3 & has7
    for t in np.nonzero(both)[0]:
        row = list(r.idx[t])
        assert row.index(3) < row.index(7)
