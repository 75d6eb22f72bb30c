"""Builds liblopt.so (HIP kernels + C ABI) for gfx950 in-tree.

    python -m learned_optimizer_step_amd.build
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "liblopt.so")
# (source, extra flags).  The apply kernels, and the one-launch step that
# runs them, assume finite values in their ReLUs (-fno-honor-nans gives a
# single v_max_f32 per ReLU).  The sources are compiled in parallel.
SOURCES = [("lopt_kernels.hip", []), ("lopt_apply.hip", ["-fno-honor-nans"]),
           ("lopt_single.hip", ["-fno-honor-nans"]), ("lopt_api.cpp", [])]
ARCH = "gfx950"

# Packed-fp32 VALU instructions are disabled for all device code.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = ("is not a recognized feature for this target", "argument unused during compilation")
    msgs = [l for l in (res.stdout + res.stderr).splitlines() if not any(x in l for x in noise)]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))


def build(verbose: bool = False, out: str = LIB, defines=()) -> str:
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    cmds, objs = [], []
    for src, extra in SOURCES:
        obj = os.path.join(objdir, os.path.splitext(src)[0] + ".o")
        cmds.append([hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-c", "-Wall",
                     "-Wno-unused-function", "-I", os.path.join(ROOT, "include"), *DEVICE_FLAGS, *extra,
                     *[f"-D{d}" for d in defines],
                     os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    with concurrent.futures.ThreadPoolExecutor(len(cmds)) as ex:
        for f in [ex.submit(_run, cmd, verbose) for cmd in cmds]:
            f.result()
    out_tmp = out + ".tmp"
    _run([hipcc(), "-shared", "-fPIC", *objs, "-o", out_tmp], verbose)
    os.replace(out_tmp, out)
    if out == LIB:
        build_microbench(verbose)
    return out


MICROBENCH = os.path.join(PKG, "lopt_microbench")


def build_microbench(verbose: bool = False) -> str:
    """The machine-figure microbenchmark (read bandwidth, matrix throughput, vector-op costs)."""
    tmp = MICROBENCH + ".tmp"
    _run([hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", *DEVICE_FLAGS, "-fno-honor-nans",
          os.path.join(CSRC, "microbench.hip"), "-o", tmp], verbose)
    os.replace(tmp, MICROBENCH)
    return MICROBENCH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
