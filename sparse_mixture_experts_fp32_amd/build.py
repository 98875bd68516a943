"""Build libmoe.so (the gfx950 kernels and the C ABI) in-tree with hipcc.

    python -m sparse_mixture_experts_fp32_amd.build

Every HIP translation unit is compiled with packed-f32 instructions disabled; the host
pass warns that it does not know that feature, which is expected.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libmoe.so")
OBJ = os.path.join(PKG, "_build")

HIP_SOURCES = ["rmsnorm.hip", "router.hip", "permute.hip", "grouped_gemm.hip", "combine.hip",
               "mx_scales.hip", "static_scratch.hip"]
CXX_SOURCES = ["moe_api.cpp"]
ARCH = os.environ.get("MOE_OFFLOAD_ARCH", "gfx950")
HIP_FLAGS = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang",
             "-packed-fp32-ops", "-munsafe-fp-atomics"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("build step failed: " + " ".join(cmd))
    noise = [ln for ln in (r.stderr or "").splitlines()
             if "packed-fp32-ops" not in ln and ln.strip()]
    if noise:
        sys.stderr.write("\n".join(noise) + "\n")


def build(verbose: bool = True, src_dir: str = CSRC, lib: str = LIB) -> str:
    """Compile the sources of ``src_dir`` into ``lib`` (defaults: this package's csrc/
    into the in-tree libmoe.so)."""
    obj_dir = OBJ if src_dir == CSRC else os.path.join(src_dir, "_build")
    os.makedirs(obj_dir, exist_ok=True)
    cc = hipcc()
    flags = ["-O3", "-std=c++17", "-fPIC", f"-I{INCLUDE}", f"-I{src_dir}"]
    objs = []
    for src in HIP_SOURCES:
        o = os.path.join(obj_dir, src + ".o")
        _run([cc, *flags, *HIP_FLAGS, "-x", "hip", "-c", os.path.join(src_dir, src), "-o", o])
        objs.append(o)
    for src in CXX_SOURCES:
        o = os.path.join(obj_dir, src + ".o")
        _run([cc, *flags, "-D__HIP_PLATFORM_AMD__", "-c", os.path.join(src_dir, src), "-o", o])
        objs.append(o)
    tmp = lib + ".tmp"
    _run([cc, "-shared", f"--offload-arch={ARCH}", "-O3", "-o", tmp, *objs])
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib}")
    return lib


if __name__ == "__main__":
    build()
