"""moe_forward_static (the layer with the library's static device scratch, for callers
that cannot allocate) against moe_forward on a caller workspace, through the C ABI: two
calls in a row, the second on fewer tokens, each equal to moe_forward bit for bit (the
same kernels on the same workspace layout) and held to the oracle's parity bar.  Its
argument checks, including the scratch-size limit, come before any device work."""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import sparse_mixture_experts_fp32_amd as M  # noqa: E402
from gpu_util import cfg_struct, device_inputs, run_forward  # noqa: E402
from moe_inputs import CONFIGS, MoEConfig, make_inputs  # noqa: E402
from oracle import moe_oracle as O  # noqa: E402
from parity import assert_outputs, check_routing  # noqa: E402

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


CASES = [
    # the Inkling decode shape (32 tokens, then 7), with its two shared experts
    CONFIGS["inkling_decode"],
    # a small sigmoid layer: 200 tokens (128-row tiles), then 32 (decode tiles)
    MoEConfig(name="static_sig_bf16", T=200, d=512, E=40, S=2, I=256, k=6, router="sigmoid",
              dtype="bf16", x_std=1.0, w_std=0.05, bias_std=0.1, zipf_s=0.0,
              zipf_hot_share=0.0, seed=42),
    # f32 softmax layer: 100 tokens, then 1
    MoEConfig(name="static_soft_f32", T=100, d=256, E=16, S=0, I=128, k=2, router="softmax",
              dtype="f32", x_std=1.0, w_std=0.05, bias_std=0.0, zipf_s=0.0,
              zipf_hot_share=0.0, seed=43),
]
SECOND = {"inkling_decode": 7, "static_sig_bf16": 32, "static_soft_f32": 1}


def static_forward(c, dev, T):
    cfg = cfg_struct(c)
    out = torch.empty((T, c.d), dtype=torch.float32, device="cuda")
    idx = torch.empty((T, c.k), dtype=torch.int32, device="cuda")
    counts = torch.empty((c.E + c.S,), dtype=torch.int32, device="cuda")
    M.moe_forward_static(cfg, T, dev["x"][:T], dev["w_router"], dev.get("sel_bias"),
                         dev.get("logit_offset"), dev["w_gate"], dev["w_up"], dev["w_down"],
                         None, out, idx, counts)
    return out, idx, counts


@pytest.mark.parametrize("c", CASES, ids=[c.name for c in CASES])
def test_static_scratch_matches_workspace_forward(c):
    inp = make_inputs(c)
    dev = device_inputs(inp, torch)
    cfg = cfg_struct(c)
    assert M.moe_workspace_size(cfg, c.T) <= M.MOE_STATIC_SCRATCH_BYTES
    for T in (c.T, SECOND[c.name]):
        log(f"[{c.name}] moe_forward_static T={T}")
        got = static_forward(c, dev, T)
        want = run_forward(c, dict(dev, x=dev["x"][:T]), torch)
        torch.cuda.synchronize()
        for g, w, what in zip(got, want, ("out", "topk_idx", "counts")):
            assert torch.equal(g, w), (c.name, T, what)
        sub = dict(inp, x=inp["x"][:T])
        ref = O.moe_forward(c.with_(T=T), sub,
                            mode="bf16_flow" if c.dtype == "bf16" else "exact")
        gidx = got[1].cpu().numpy()
        excl = check_routing(gidx, ref.routing, c.E)
        y = ref.y.copy()
        if excl.any():
            t = np.nonzero(excl)[0]
            y[t] = O.moe_forward(c.with_(T=T), sub, mode="bf16_flow" if c.dtype == "bf16"
                                 else "exact", tokens=t, forced_idx=gidx[t]).y
        mx, mn = assert_outputs(got[0].cpu().numpy(), y, f"{c.name} static T={T}")
        log(f"[{c.name}] T={T}: bit-identical to moe_forward; max rel {mx:.2e}, "
            f"mean rel {mn:.2e}")


def test_static_scratch_limit_is_checked_before_any_device_work():
    c = CONFIGS["inkling_prefill"]
    cfg = cfg_struct(c)
    assert M.moe_workspace_size(cfg, c.T) > M.MOE_STATIC_SCRATCH_BYTES
    A = 0x7F0000000000
    with pytest.raises(M.MoEError) as ei:
        M.moe_forward_static(cfg, c.T, A, A, None, None, A, A, A, None, A, None, None)
    assert ei.value.status == M.MOE_ERR_WORKSPACE
