"""The C ABI layer (argument checks, workspace layout, launch sequence) built for the host
with AddressSanitizer and UndefinedBehaviorSanitizer, with the kernel launchers replaced
by stand-ins that touch every byte the kernels would read or write (tests/sanitize/).
No GPU and no HIP runtime are involved; the driver calls every entry point on exact-size
host buffers and checks every status."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "sparse_mixture_experts_fp32_amd", "csrc")
SAN = os.path.join(HERE, "sanitize")

CXX = shutil.which("g++")
pytestmark = pytest.mark.skipif(CXX is None, reason="needs g++")


def build_and_run(api_source, out_dir):
    exe = os.path.join(out_dir, "abi_sanitize")
    cmd = [CXX, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__",
           "-I/opt/rocm/include", f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}",
           api_source, os.path.join(SAN, "abi_stubs.cpp"), os.path.join(SAN, "abi_driver.cpp"),
           "-o", exe]
    b = subprocess.run(cmd, capture_output=True, text=True)
    assert b.returncode == 0, b.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    return subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)


def test_c_abi_under_asan_and_ubsan(tmp_path):
    r = build_and_run(os.path.join(CSRC, "moe_api.cpp"), str(tmp_path))
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-4000:])
    assert "all shapes ok" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr


def test_planted_layout_overlap_is_caught(tmp_path):
    """A workspace layout that sizes the intermediate h without its row pad (a plausible
    mistake) lets h spill into the expert-row region: the stand-ins report it."""
    src = open(os.path.join(CSRC, "moe_api.cpp")).read()
    good = "L.h = take(esize * m.R * moe::h_pitch(m.I));"
    assert good in src
    planted = tmp_path / "moe_api_planted.cpp"
    planted.write_text(src.replace(good, "L.h = take(esize * m.R * m.I);"))
    r = build_and_run(str(planted), str(tmp_path))
    assert r.returncode != 0
    assert "overlaps" in r.stderr or "AddressSanitizer" in r.stderr
