"""The library's host planner under AddressSanitizer and UndefinedBehaviorSanitizer.

lopt_api.cpp (validation, planning, the workspace layout, the uploads between
steps) is compiled for the CPU with the host compiler and both sanitizers,
linked with host stand-ins of the HIP calls it makes and of the two launch
functions (tests/sanitizer/hip_host_stub.cpp: the stand-ins check every index
of the plan and write every workspace range the kernels write), and driven
through its C ABI by tests/sanitizer/planner_main.cpp: argument validation, the
edges of the size range (1 x 1, 1 x (2^31 - 1), 2 x (2^28 - 1),
2^16 x (2^15 - 1)), 150 seeded random lists, and the ViT-B/16, GPT-2 355M,
Llama-style and ragged 10,000-tensor lists, each workspace allocated with
exactly the size the library reports.  No device is used.
"""
import os
import shutil
import subprocess

import pytest

from learned_optimizer_step_amd import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitizer")
HIP_INCLUDE = "/opt/rocm/include"


@pytest.fixture(scope="module")
def planner_binary(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None or not os.path.exists(os.path.join(HIP_INCLUDE, "hip", "hip_runtime_api.h")):
        pytest.skip("needs g++ and the HIP headers")
    out = str(tmp_path_factory.mktemp("planner") / "planner_sanitized")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-D__HIP_PLATFORM_AMD__", "-I", HIP_INCLUDE, "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "learned_optimizer_step_amd", "csrc", "lopt_api.cpp"),
           os.path.join(SAN, "hip_host_stub.cpp"), os.path.join(SAN, "planner_main.cpp"), "-o", out]
    res = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert res.returncode == 0, res.stderr[-3000:]
    return out


def test_planner_is_clean_under_sanitizers(planner_binary, tmp_path):
    lists = []
    for key in ("vit_b16", "gpt2_355m", "llama1b", "ragged10k"):
        path = tmp_path / f"{key}.txt"
        path.write_text("".join(f"{t.rows} {t.cols}\n" for t in W.get_workload(key).tensors))
        lists.append(str(path))
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    res = subprocess.run([planner_binary, *lists], capture_output=True, text=True, timeout=900, env=env)
    assert res.returncode == 0, (res.stdout[-2000:], res.stderr[-4000:])
    assert "0 failures" in res.stdout and "Sanitizer" not in res.stderr, res.stderr[-2000:]
    assert "160 lists" in res.stdout, res.stdout
