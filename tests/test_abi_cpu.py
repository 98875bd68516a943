"""The C ABI on the host: the library loads, exports every function include/moe.h
declares, sizes workspaces, and rejects bad arguments before touching the GPU.  No
compute call is made."""
import ctypes
import os

import pytest

import sparse_mixture_experts_fp32_amd as M
from moe_inputs import CONFIGS, CONFIG_ORDER

pytestmark = pytest.mark.skipif(not os.path.exists(M.LIB_PATH),
                                reason="libmoe.so not built (run __graft_entry__.build())")

# Plausible-looking aligned device addresses: every call below fails validation before
# any of them would be dereferenced or handed to HIP.
A = 0x7F0000000000


def cfg_of(c, **kw):
    args = dict(d_model=c.d, n_experts=c.E, d_ff=c.I, top_k=c.k, n_shared=c.S,
                router=c.router, dtype=c.dtype)
    args.update(kw)
    return M.make_config(**args)


def test_binding_parameter_counts_match_the_header():
    from sparse_mixture_experts_fp32_amd import moe as binding
    binding.load_library()
    counts = binding.header_param_counts()
    bound = binding.ARGTYPES
    assert set(bound) <= set(counts)
    for name, n in bound.items():
        assert counts[name] == n, (name, counts[name], n)
    # every declared entry point is bound
    assert set(counts) - set(bound) == {"moe_status_str"}


def test_library_exports_every_declared_function():
    lib = M.load_library()
    names = M.header_functions()
    assert set(names) == {"moe_status_str", "moe_workspace_size", "moe_route", "moe_permute",
                          "moe_grouped_swiglu", "moe_combine", "moe_forward", "moe_rmsnorm",
                          "moe_forward_rmsnorm", "moe_grouped_swiglu_mxfp4",
                          "moe_forward_mxfp4", "moe_mxfp4_scales_bytes",
                          "moe_mxfp4_pack_scales", "moe_forward_static"}
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings():
    for s in range(5):
        assert M.status_str(s).startswith("MOE_")
    assert "UNKNOWN" in M.status_str(99)


@pytest.mark.parametrize("name", CONFIG_ORDER)
def test_workspace_size_covers_the_intermediates(name):
    c = CONFIGS[name]
    cfg = cfg_of(c)
    ws = M.moe_workspace_size(cfg, c.T)
    esize = 2 if c.dtype == "bf16" else 4
    rows = c.T * (c.k + c.S)
    assert ws >= rows * c.d * 4 + rows * c.I * esize       # y_rows (f32) + h
    assert M.moe_workspace_size(cfg, 0) < ws
    assert M.moe_workspace_size(cfg, c.T + 1) >= ws


@pytest.mark.parametrize("bad,status", [
    (dict(top_k=0), M.MOE_ERR_ARG),
    (dict(top_k=300), M.MOE_ERR_ARG),
    (dict(n_shared=-1), M.MOE_ERR_ARG),
    (dict(router=7), M.MOE_ERR_ARG),
    (dict(dtype=5), M.MOE_ERR_ARG),
    (dict(route_scale=0.0), M.MOE_ERR_ARG),
    (dict(route_scale=float("nan")), M.MOE_ERR_ARG),
    (dict(d_model=6000), M.MOE_ERR_UNSUPPORTED),
    (dict(d_ff=3000), M.MOE_ERR_UNSUPPORTED),
    (dict(top_k=33, n_experts=256), M.MOE_ERR_UNSUPPORTED),
    (dict(n_experts=1020, n_shared=8), M.MOE_ERR_UNSUPPORTED),
])
def test_config_validation(bad, status):
    cfg = cfg_of(CONFIGS["inkling_decode"], **bad)
    with pytest.raises(M.MoEError) as ei:
        M.moe_workspace_size(cfg, 32)
    assert ei.value.status == status


def _largest_tokens(d, I, A_, es):
    # Largest T with T (k + S) max(d, I) <= 2^31 elements, T d es < 2^31 bytes (x) and
    # T (k + S) (I + 64) es < 2^31 bytes (the padded intermediate), by direct search.
    def fits(T):
        R = T * A_
        return (R * max(d, I) <= 1 << 31 and T * d * es < 1 << 31
                and R * (I + 64) * es < 1 << 31)
    lo, hi = 1, 1 << 40
    while hi - lo > 1:
        mid = (lo + hi) // 2
        lo, hi = (mid, hi) if fits(mid) else (lo, mid)
    return lo


@pytest.mark.parametrize("name,A_", [("inkling_prefill", None), ("qwen38", None),
                                     ("tiny_fp32", 1), ("tiny_fp32", 32)])
def test_token_count_limited_by_32_bit_offsets(name, A_):
    # The kernels address the grouped rows with 32-bit element offsets and read x and the
    # intermediate h through 32-bit byte ranges; the first token count past any of these
    # limits is refused.
    c = CONFIGS[name]
    top_k = A_ if A_ is not None else c.k
    n_experts = max(c.E, top_k)
    cfg = cfg_of(c, top_k=top_k, n_experts=n_experts)
    es = 4 if c.dtype == "f32" else 2
    t_max = _largest_tokens(c.d, c.I, top_k + c.S, es)
    assert M.moe_workspace_size(cfg, t_max) > 0
    with pytest.raises(M.MoEError) as ei:
        M.moe_workspace_size(cfg, t_max + 1)
    assert ei.value.status == M.MOE_ERR_UNSUPPORTED


def test_softmax_router_takes_ungated_shared_experts_but_no_scale():
    c = CONFIGS["qwen38"]
    # Ungated shared experts are accepted (up to 8); they add T rows each.
    base = M.moe_workspace_size(cfg_of(c), 8)
    assert M.moe_workspace_size(cfg_of(c, n_shared=1), 8) > base
    with pytest.raises(M.MoEError) as ei:
        M.moe_workspace_size(cfg_of(c, n_shared=9), 8)
    assert ei.value.status == M.MOE_ERR_UNSUPPORTED
    with pytest.raises(M.MoEError):
        M.moe_workspace_size(cfg_of(c, route_scale=2.0), 8)
    with pytest.raises(M.MoEError):
        M.moe_workspace_size(cfg_of(c, bias_on_logits=True), 8)


def test_entry_points_validate_before_launch():
    c = CONFIGS["inkling_decode"]
    cfg = cfg_of(c)
    T = c.T
    need = M.moe_workspace_size(cfg, T)

    def status(fn, *args):
        with pytest.raises(M.MoEError) as ei:
            fn(*args, stream=0)
        return ei.value.status

    # null / misaligned pointers
    assert status(M.moe_route, cfg, T, None, A, None, None, A, A, A, need) == M.MOE_ERR_ARG
    assert status(M.moe_route, cfg, T, A + 2, A, None, None, A, A, A, need) == M.MOE_ERR_ARG
    assert status(M.moe_route, cfg, T, A, A, None, None, A, A, A + 64, need) == M.MOE_ERR_ARG
    # workspace too small
    assert status(M.moe_route, cfg, T, A, A, None, None, A, A, A, need - 1) == \
        M.MOE_ERR_WORKSPACE
    assert status(M.moe_permute, cfg, T, A, A, A, A, A, A, 16) == M.MOE_ERR_WORKSPACE
    assert status(M.moe_permute, cfg, T, A, None, A, A, A, A, need) == M.MOE_ERR_ARG
    assert status(M.moe_grouped_swiglu, cfg, T, A, A, A, A, A, A, A, A, 0) == \
        M.MOE_ERR_WORKSPACE
    assert status(M.moe_grouped_swiglu, cfg, T, A, A, A, A, A + 8, A, A, A, need) == \
        M.MOE_ERR_ARG
    assert status(M.moe_combine, cfg, T, A, A, None, None, A) == M.MOE_ERR_ARG
    assert status(M.moe_combine, cfg, T, A, A, A, A + 4, A) == M.MOE_ERR_ARG
    assert status(M.moe_forward, cfg, T, A, A, None, None, A, A, A, None, A, None, None,
                  A, 1) == M.MOE_ERR_WORKSPACE
    assert status(M.moe_forward, cfg, -1, A, A, None, None, A, A, A, None, A, None, None,
                  A, need) == M.MOE_ERR_ARG
    # a selection bias only exists for the sigmoid router
    q = CONFIGS["qwen38"]
    qcfg = cfg_of(q)
    qneed = M.moe_workspace_size(qcfg, 8)
    assert status(M.moe_route, qcfg, 8, A, A, A, None, A, A, A, qneed) == M.MOE_ERR_ARG


def test_rmsnorm_entry_points_validate_before_launch():
    c = CONFIGS["inkling_decode"]
    cfg = cfg_of(c)
    need = M.moe_workspace_size(cfg, c.T)

    def status(fn, *args):
        with pytest.raises(M.MoEError) as ei:
            fn(*args, stream=0)
        return ei.value.status

    assert status(M.moe_rmsnorm, cfg, 4, A, A, 0.0, 0, A) == M.MOE_ERR_ARG        # eps
    assert status(M.moe_rmsnorm, cfg, 4, A, A, float("nan"), 0, A) == M.MOE_ERR_ARG
    assert status(M.moe_rmsnorm, cfg, 4, A, A, 1e-6, 2, A) == M.MOE_ERR_ARG        # flag
    assert status(M.moe_rmsnorm, cfg, 4, None, A, 1e-6, 0, A) == M.MOE_ERR_ARG
    assert status(M.moe_rmsnorm, cfg, 4, A + 8, A, 1e-6, 0, A) == M.MOE_ERR_ARG
    wide = cfg_of(c, d_model=16640)
    assert status(M.moe_rmsnorm, wide, 4, A, A, 1e-6, 0, A) == M.MOE_ERR_UNSUPPORTED
    assert status(M.moe_forward_rmsnorm, cfg, c.T, A, A, 1e-6, 1, A, None, None, A, A, A,
                  None, A, None, None, A, need - 1) == M.MOE_ERR_WORKSPACE
    assert status(M.moe_forward_rmsnorm, cfg, c.T, A, None, 1e-6, 1, A, None, None, A, A,
                  A, None, A, None, None, A, need) == M.MOE_ERR_ARG
    # T = 0 is a no-op
    M.moe_rmsnorm(cfg, 0, None, None, 1e-6, 0, None, stream=0)


def test_mxfp4_entry_points_validate_before_launch():
    c = CONFIGS["inkling_decode"]
    cfg = cfg_of(c)
    need = M.moe_workspace_size(cfg, c.T)
    q = [A, A + 16, A, A + 16, A, A + 16]       # codes and packed scales 16-byte aligned

    def status(fn, *args):
        with pytest.raises(M.MoEError) as ei:
            fn(*args, stream=0)
        return ei.value.status

    f32 = cfg_of(c, dtype="f32")
    assert status(M.moe_grouped_swiglu_mxfp4, f32, c.T, A, A, A, *q, A, A, A, A, A,
                  need) == M.MOE_ERR_UNSUPPORTED
    assert status(M.moe_grouped_swiglu_mxfp4, cfg, c.T, A, A, A, None, *q[1:], A, A, A, A,
                  A, need) == M.MOE_ERR_ARG
    assert status(M.moe_grouped_swiglu_mxfp4, cfg, c.T, A, A, A, A + 8, *q[1:], A, A, A,
                  A, A, need) == M.MOE_ERR_ARG                  # misaligned codes
    assert status(M.moe_grouped_swiglu_mxfp4, cfg, c.T, A, A, A, A, A + 1, *q[2:], A, A,
                  A, A, A, need) == M.MOE_ERR_ARG               # misaligned packed scales
    assert status(M.moe_grouped_swiglu_mxfp4, cfg, c.T, A, A, A, *q, None, A, A, A, A,
                  need) == M.MOE_ERR_ARG                        # S = 2 needs shared weights
    assert status(M.moe_forward_mxfp4, cfg, c.T, A, A, None, None, *q, A, A, A, None, A,
                  None, None, A, need - 1) == M.MOE_ERR_WORKSPACE


@pytest.mark.parametrize("E,N,K", [(1, 64, 32), (256, 3072, 6144), (256, 6144, 3072),
                                   (16, 384, 256), (16, 256, 384), (6, 128, 128)])
def test_mxfp4_scales_bytes(E, N, K):
    # one 512-byte record per expert, 64 rows of N and 8 MX blocks (256 elements) of K,
    # the last record along K zero-padded
    records_k = -(-(K // 32) // 8)
    assert M.moe_mxfp4_scales_bytes(E, N, K) == E * (N // 64) * records_k * 512
    assert M.moe_mxfp4_scales_bytes(E, N, K) >= E * N * (K // 32)


@pytest.mark.parametrize("E,N,K", [(2, 64, 256), (3, 128, 384), (1, 192, 32)])
def test_packed_scale_order_matches_the_header_formula(E, N, K):
    # include/moe.h: packed[(((e * N/64 + nb) * KR + kr) * 64 + r) * 8 + j]
    #                  = scale[e, 64 nb + r, 8 kr + j], zero where 8 kr + j >= K/32
    from gpu_util import packed_scale_order
    import numpy as np
    KB, KR = K // 32, -(-(K // 32) // 8)
    s = np.random.default_rng(E * N + K).integers(0, 256, size=(E, N, KB), dtype=np.uint8)
    want = np.zeros(M.moe_mxfp4_scales_bytes(E, N, K), np.uint8)
    for e in range(E):
        for nb in range(N // 64):
            for kr in range(KR):
                for r in range(64):
                    for j in range(8):
                        if 8 * kr + j < KB:
                            want[(((e * (N // 64) + nb) * KR + kr) * 64 + r) * 8 + j] = \
                                s[e, 64 * nb + r, 8 * kr + j]
    np.testing.assert_array_equal(packed_scale_order(s), want)


def test_mxfp4_pack_validates_before_launch():
    def status(fn, *args, **kw):
        with pytest.raises(M.MoEError) as ei:
            fn(*args, **kw)
        return ei.value.status

    for E, N, K in [(0, 64, 32), (1, 0, 32), (1, 64, 0), (-1, 64, 32)]:
        assert status(M.moe_mxfp4_scales_bytes, E, N, K) == M.MOE_ERR_ARG
        assert status(M.moe_mxfp4_pack_scales, E, N, K, A, A, stream=0) == M.MOE_ERR_ARG
    for E, N, K in [(1, 96, 32), (1, 64, 48), (1, 32, 256)]:
        assert status(M.moe_mxfp4_scales_bytes, E, N, K) == M.MOE_ERR_UNSUPPORTED
        assert status(M.moe_mxfp4_pack_scales, E, N, K, A, A,
                      stream=0) == M.MOE_ERR_UNSUPPORTED
    # one expert's packed scales must stay below 2 GiB (32-bit offsets in the kernels)
    assert status(M.moe_mxfp4_scales_bytes, 1, 1 << 20, 1 << 16) == M.MOE_ERR_UNSUPPORTED
    assert status(M.moe_mxfp4_pack_scales, 1, 64, 32, None, A, stream=0) == M.MOE_ERR_ARG
    assert status(M.moe_mxfp4_pack_scales, 1, 64, 32, A, None, stream=0) == M.MOE_ERR_ARG
    assert status(M.moe_mxfp4_pack_scales, 1, 64, 32, A, A + 8, stream=0) == M.MOE_ERR_ARG


def test_zero_tokens_is_a_no_op():
    cfg = cfg_of(CONFIGS["inkling_decode"])
    # T = 0 returns before any pointer is looked at and before any HIP call.
    M.moe_forward(cfg, 0, None, None, None, None, None, None, None, None, None, None, None,
                  None, 0, stream=0)
    M.moe_route(cfg, 0, None, None, None, None, None, None, None, 0, stream=0)
    M.moe_permute(cfg, 0, None, None, None, None, None, None, 0, stream=0)
    M.moe_grouped_swiglu(cfg, 0, None, None, None, None, None, None, None, None, 0, stream=0)
    M.moe_combine(cfg, 0, None, None, None, None, None, stream=0)
    M.moe_grouped_swiglu_mxfp4(cfg, 0, None, None, None, *([None] * 6), None, None, None,
                               None, None, 0, stream=0)
    M.moe_forward_mxfp4(cfg, 0, None, None, None, None, *([None] * 6), None, None, None,
                        None, None, None, None, None, 0, stream=0)
    M.moe_forward_rmsnorm(cfg, 0, None, None, 1e-6, 0, None, None, None, None, None, None,
                          None, None, None, None, None, 0, stream=0)


def test_binding_refuses_host_and_strided_tensors():
    # A host tensor's address handed to a kernel would fault the GPU; the binding refuses
    # it (and non-contiguous views) before calling into the library.
    torch = pytest.importorskip("torch")
    c = CONFIGS["inkling_decode"]
    cfg = cfg_of(c)
    need = M.moe_workspace_size(cfg, c.T)
    x = torch.zeros((c.T, c.d), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU tensor"):
        M.moe_route(cfg, c.T, x, A, None, None, A, A, A, need, stream=0)
    with pytest.raises(ValueError, match="GPU tensor"):
        M.moe_combine(cfg, c.T, A, A, A, None, x.float().t(), stream=0)


def test_binding_checks_dtype_and_extent_of_every_tensor():
    # A tensor of the wrong element type, or shorter than the extent the header gives for
    # the config and T, would let a kernel read past its end: the binding names the
    # argument and raises before calling into the library.  Meta tensors carry dtype and
    # size without memory; the other arguments are plain addresses, which pass unchecked.
    torch = pytest.importorskip("torch")
    c = CONFIGS["inkling_decode"]
    cfg = cfg_of(c)
    G, R = c.E + c.S, c.T * (c.k + c.S)
    need = M.moe_workspace_size(cfg, c.T)

    def t(shape, dt=torch.bfloat16):
        return torch.empty(shape, dtype=dt, device="meta")

    def err(match, fn, *args):
        with pytest.raises(ValueError, match=match):
            fn(*args, stream=0)

    x = t((c.T, c.d))
    wg, wd = t((G, c.I, c.d)), t((G, c.d, c.I))
    err(r"^x: expected torch.bfloat16", M.moe_route, cfg, c.T, x.float(), A, None, None,
        A, A, A, need)
    err(r"^w_router: holds", M.moe_route, cfg, c.T, A, t((G - 1, c.d)), None, None, A, A,
        A, need)
    err(r"^sel_bias: expected torch.float32", M.moe_route, cfg, c.T, A, A, t((c.E,)), None,
        A, A, A, need)
    err(r"^weights: holds", M.moe_route, cfg, c.T, A, A, None, None, A,
        t((c.T, c.k), torch.float32), A, need)
    err(r"^ws: ", M.moe_route, cfg, c.T, A, A, None, None, A, A,
        t((need - 1,), torch.uint8), need)
    err(r"^counts: expected torch.int32", M.moe_permute, cfg, c.T, A,
        t((G,), torch.int64), A, A, A, A, need)
    err(r"^offsets: holds", M.moe_permute, cfg, c.T, A, A, t((G,), torch.int32), A, A, A,
        need)
    err(r"^w_up: holds", M.moe_grouped_swiglu, cfg, c.T, A, A, A, A, wg[:-1], A, A, A,
        need)
    err(r"^y_rows: expected torch.float32", M.moe_grouped_swiglu, cfg, c.T, A, A, A, A, A,
        A, t((R, c.d)), A, need)
    err(r"^slot_row: holds", M.moe_combine, cfg, c.T, A, t((R - 1,), torch.int32), A,
        None, A)
    err(r"^residual: expected torch.float32", M.moe_combine, cfg, c.T, A, A, A,
        t((c.T, c.d)), A)
    err(r"^w_down: holds", M.moe_forward, cfg, c.T, A, A, None, None, A, A,
        wd[:, :, :-1], None, A, None, None, A, need)
    err(r"^counts_out: holds", M.moe_forward, cfg, c.T, A, A, None, None, A, A, A, None, A,
        None, t((c.E,), torch.int32), A, need)
    err(r"^gain: expected torch.bfloat16", M.moe_rmsnorm, cfg, c.T, A,
        t((c.d,), torch.float32), 1e-6, 0, A)
    # MXFP4: codes [E, N, K/2] and packed scales of the header's size.
    s = t((M.moe_mxfp4_scales_bytes(c.E, c.I, c.d) - 1,), torch.uint8)
    err(r"^ws_up: holds", M.moe_grouped_swiglu_mxfp4, cfg, c.T, A, A, A, A, A, A, s, A, A,
        A, A, A, A, A, need)
    err(r"^wq_down: expected torch.uint8", M.moe_grouped_swiglu_mxfp4, cfg, c.T, A, A, A,
        A, A, A, A, t((c.E, c.d, c.I // 2)), A, A, A, A, A, A, need)
    err(r"^w_gate_shared: expected torch.bfloat16", M.moe_forward_mxfp4, cfg, c.T, A, A,
        None, None, A, A, A, A, A, A, t((c.S, c.I, c.d), torch.float32), A, A, None, A,
        None, None, A, need)
    # Tensors of the right type and extent pass and stop at the device check.
    err("GPU tensor", M.moe_route, cfg, c.T, x, A, None, None, A, A, A, need)
    err("GPU tensor", M.moe_forward, cfg, c.T, A, A, None, None, wg, A, A, None, A, None,
        None, A, need)


def test_config_struct_layout_matches_header():
    assert ctypes.sizeof(M.moe_config_t) == 9 * 4


C_PROGRAM = r"""
#include <stdio.h>
#include "moe.h"
int main(void) {
  moe_config_t c = {6144, 256, 3072, 6, 2, MOE_ROUTER_SIGMOID_SHARED, MOE_BF16, 0, 8.0f};
  size_t bytes = 0;
  moe_status_t s = moe_workspace_size(&c, 32, &bytes);
  printf("%d %zu\n", (int)s, bytes);
  c.top_k = 300;   /* more than n_experts */
  s = moe_workspace_size(&c, 32, &bytes);
  printf("%d %s\n", (int)s, moe_status_str(s));
  return 0;
}
"""


def test_header_is_plain_c_and_links():
    # The boundary is a C ABI: a C99 translation unit includes moe.h, links libmoe.so and
    # calls host-only entry points (no GPU needed).
    import shutil
    import subprocess
    import tempfile
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    libdir = os.path.join(root, "sparse_mixture_experts_fp32_amd")
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    with tempfile.TemporaryDirectory() as d:
        src, exe = os.path.join(d, "abi.c"), os.path.join(d, "abi")
        with open(src, "w") as f:
            f.write(C_PROGRAM)
        subprocess.run([gcc, "-std=c99", "-Wall", "-Werror=implicit-function-declaration",
                        "-D__HIP_PLATFORM_AMD__", f"-I{root}/include", f"-I{rocm}/include",
                        src, f"-L{libdir}", "-lmoe", f"-Wl,-rpath,{libdir}", "-o", exe],
                       check=True, capture_output=True, text=True, timeout=120)
        out = subprocess.run([exe], check=True, capture_output=True, text=True,
                             timeout=60).stdout.split("\n")
    c = CONFIGS["inkling_decode"]
    status, nbytes = map(int, out[0].split())
    assert status == M.MOE_OK and nbytes == M.moe_workspace_size(cfg_of(c), 32)
    assert out[1].startswith(f"{M.MOE_ERR_ARG} MOE_ERR_ARG")
