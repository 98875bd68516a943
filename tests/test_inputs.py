"""The seeded input generator: determinism, independence of streams, value recipe."""
import numpy as np

from moe_inputs import CONFIGS, fill_expert_tensor, make_expert, make_inputs, make_x
from moe_inputs.generate import make_logit_offset, zipf_ranks


def test_same_seed_same_bytes():
    cfg = CONFIGS["tiny_fp32"]
    a, b = make_inputs(cfg), make_inputs(cfg)
    for key in ("x", "w_router", "w_gate", "w_up", "w_down"):
        assert a[key].tobytes() == b[key].tobytes()


def test_experts_regenerate_independently_in_any_order():
    cfg = CONFIGS["tiny_fp32"].with_(E=6)
    full = fill_expert_tensor(cfg, "w_up")
    part = np.zeros_like(full)
    fill_expert_tensor(cfg, "w_up", out=part, experts=[4, 1, 5])
    for e in (1, 4, 5):
        assert (part[e] == full[e]).all()
        assert (make_expert(cfg, "w_up", e) == full[e]).all()
    assert not (full[0] == full[1]).all()


def test_x_prefix_is_the_same_batch():
    cfg = CONFIGS["inkling_decode"].with_(d=64)
    big = make_x(cfg, T=2500)
    small = make_x(cfg, T=32)
    assert (big[:32] == small).all()


def test_value_recipe_statistics():
    cfg = CONFIGS["inkling_decode"].with_(d=512, E=200, I=64)
    inp = make_inputs(cfg)
    f = lambda u: (u.astype(np.uint32) << 16).view(np.float32)  # noqa: E731
    assert inp["x"].dtype == np.uint16
    assert abs(f(inp["x"]).std() - 1.0) < 0.02
    assert abs(f(inp["w_gate"]).std() - 0.02) < 0.0005
    assert abs(inp["sel_bias"].std() - 0.1) < 0.03
    assert inp["logit_offset"] is None


def test_zipf_offset_form():
    cfg = CONFIGS["inkling_skewed"]
    r = zipf_ranks(cfg)
    assert sorted(r.tolist()) == list(range(1, cfg.E + 1))
    o = make_logit_offset(cfg, a=1.0)
    np.testing.assert_allclose(o, -1.2 * np.log(r), rtol=1e-6)
    assert o[np.argmin(r)] == 0.0
