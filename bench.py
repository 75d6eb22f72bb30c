"""Throughput of the small_fc_lopt optimizer step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload vit_b16]

A step is one lopt_step over the whole parameter list (row/column sums,
moving averages, statistics, finalize, apply).  Inputs (parameters, state,
gradients) are resident in HBM before the timed region; the same gradients
are reused for every timed step.  Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def flop_per_elem(n_feat: int = 28) -> int:
    """MLP FLOP per element with the step features folded into the first bias."""
    return 2 * (n_feat * 32 + 32 * 32 + 32 * 2)


PEAK_FP32_MFMA_TFLOPS = 157.3                      # MI355X dense fp32 matrix
PEAK_FP32_VALU_TFLOPS = 78.6                       # 256 CU x 4 SIMD x 16 lanes x 2 x 2.4 GHz (no packed fp32)
PEAK_BF16_MFMA_TFLOPS = 2500.0                     # MI355X dense bf16 matrix
PEAK_FP16_MFMA_TFLOPS = 2500.0                     # MI355X dense fp16 matrix
X6_PRODUCTS = 6                                    # bf16 piece products per fp32 product (bf16x6 path)
X3_PRODUCTS = 3                                    # fp16 piece products per fp32 product (fp16x3 path)
PEAK_HBM_GBS = 8000.0
# ViT-B/16 step of small_fc_lopt with the fused CUDA kernels on the PyLO page
# ("Benchmark results" > step-time table): 99.59 ms for 86,563,584 parameters.
PAGE_VIT_GPARAMS_PER_S = 86_563_584 / 99.59e-3 / 1e9


def log(msg):
    print(msg, file=sys.stderr, flush=True)


# Sources of the apply kernel; the committed HBM-traffic figure is only valid
# for the code it was measured on (comments and blank lines do not count).
APPLY_SOURCES = ("learned_optimizer_step_amd/csrc/lopt_apply.hip", "learned_optimizer_step_amd/csrc/lopt_device.h",
                 "learned_optimizer_step_amd/csrc/lopt_internal.h")


def code_text(src: str) -> str:
    """C++ source without comments, trailing blanks and empty lines."""
    import re
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    lines = (re.sub(r"//.*$", "", line).rstrip() for line in src.splitlines())
    return "\n".join(line for line in lines if line.strip())


def apply_sources_sha() -> str:
    import hashlib
    h = hashlib.sha256()
    for p in APPLY_SOURCES:
        with open(os.path.join(ROOT, p)) as f:
            h.update(code_text(f.read()).encode())
    return h.hexdigest()[:16]


def committed_traffic(workload: str, kernel: str = "k_apply_mfma"):
    """HBM bytes per launch of ``kernel`` from the rocprofv3 FETCH_SIZE/WRITE_SIZE
    summary in profiles/, or None when absent or measured on other sources."""
    path = os.path.join(ROOT, "profiles", f"{workload}_hbm_traffic.md")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        for line in f:
            if not line.startswith("bench-traffic:"):
                continue
            kv = dict(x.split("=", 1) for x in line.split()[1:])
            if kv.get("kernel") == kernel and kv.get("workload") == workload:
                return int(kv["bytes"]) if kv.get("sources_sha256") == apply_sources_sha() else None
    return None


def cpu_baseline(blocks: int = 7):
    """The oracle on the first ``blocks`` ViT-B/16 transformer blocks, one step, on host cores."""
    import numpy as np
    from threadpoolctl import threadpool_info, threadpool_limits

    import oracle
    from learned_optimizer_step_amd import workloads as W

    cores = len(os.sched_getaffinity(0))
    threads = min(cores, 16)
    w = W.get_workload("vit_b16")
    prefixes = tuple(f"blocks.{b}." for b in range(blocks))
    idx = [i for i, t in enumerate(w.tensors) if t.name.startswith(prefixes)]
    ps = [W.param_init(w, i) for i in idx]
    gs = [W.grad_at(w, i, 1) for i in idx]
    sts = [W.state_init(w, i) for i in idx]
    n = sum(w.tensors[i].n for i in idx)
    mlp = W.mlp_weights()
    with threadpool_limits(limits=threads):
        t0 = time.perf_counter()
        oracle.step(ps, gs, sts, 1, mlp, oracle.Hyper())
        dt = time.perf_counter() - t0
    return {"value": n / dt / 1e9, "unit": "G params/s", "cores": threads, "kind": "oracle",
            "sample": f"ViT-B/16 blocks 0-{blocks - 1} ({len(idx)} tensors, {n} params), 1 step, "
                      f"fp64 NumPy, {threads} BLAS threads, {dt:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="vit_b16")
    ap.add_argument("--impl", default="auto", choices=["auto", "valu", "mfma", "bf16x6", "fp16x3"])
    ap.add_argument("--n-feat", type=int, default=28, choices=(28, 19),
                    help="per-element features: 28 (small_fc_lopt) or 19 (the VeLO-shaped variant)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-fp32-compare", action="store_true",
                    help="with a split MLP path (fp16x3, bf16x6), skip timing the fp32 matrix path and the other "
                         "split path on the same inputs")
    ap.add_argument("--peaks", action="store_true",
                    help="also run the machine-figure microbenchmark and include it as measured_peaks")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="after the timed steps, run one plain 1 GiB device copy (reference for HBM counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the library has no "
              f"multi-GPU path", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from learned_optimizer_step_amd import lopt as L
    from learned_optimizer_step_amd import workloads as W

    impl = {"auto": L.LOPT_MLP_AUTO, "valu": L.LOPT_MLP_VALU, "mfma": L.LOPT_MLP_MFMA,
            "bf16x6": L.LOPT_MLP_BF16X6, "fp16x3": L.LOPT_MLP_FP16X3}[args.impl]
    w = W.get_workload(args.workload)
    log(f"[bench] {w.key}: {len(w.tensors)} tensors, {w.n_params} params; generating inputs")
    dev = torch.device("cuda:0")
    params, grads = [], []
    for i, t in enumerate(w.tensors):
        params.append(torch.from_numpy(W.param_init(w, i).reshape(t.shape)).to(dev))
        grads.append(torch.from_numpy(W.grad_at(w, i, 1).reshape(t.shape)).to(dev))
    cfg = L.config_from(mlp_impl=impl, n_feat=args.n_feat)
    opt = L.LOpt(params, W.mlp_weights(n_feat=args.n_feat), cfg)
    if w.prewarm_std is not None:
        for i in range(len(w.tensors)):
            st = W.state_init(w, i)
            v = opt.state_views(i)
            for k in ("m", "v", "r", "c"):
                v[k].copy_(torch.from_numpy(st[k]))
    impl = L.lopt_get_mlp_impl(opt.handle)   # "auto" resolved for these weights
    torch.cuda.synchronize()
    log(f"[bench] warmup {args.warmup} steps")
    for _ in range(args.warmup):
        opt.step(grads)
    torch.cuda.synchronize()

    nk = L.LOPT_N_KERNELS
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(nk + 1)] for _ in range(args.steps)]
    stream = torch.cuda.current_stream(dev)
    for evs in events:          # torch creates the HIP event on first record
        for e in evs:
            e.record(stream)
    log(f"[bench] timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        L.lopt_set_timing_events(opt.handle, [e.cuda_event for e in events[k]])
        opt.step(grads)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    L.lopt_set_timing_events(opt.handle, [])
    ms = (t1 - t0) * 1e3 / args.steps
    kern = np.array([[events[k][j].elapsed_time(events[k][j + 1]) for j in range(nk)]
                     for k in range(args.steps)])
    kern_ms = kern.mean(axis=0)
    per_step = np.array([events[k][0].elapsed_time(events[k][nk]) for k in range(args.steps)])
    def time_path(path_impl, k2=20):
        """The same optimizer and inputs for k2 more steps with another apply kernel."""
        L.lopt_set_config(opt.handle, L.config_from(mlp_impl=path_impl, n_feat=args.n_feat))
        for _ in range(2):
            opt.step(grads)
        ev2 = [[torch.cuda.Event(enable_timing=True) for _ in range(nk + 1)] for _ in range(k2)]
        for evs in ev2:
            for e in evs:
                e.record(stream)
        torch.cuda.synchronize()
        t2 = time.perf_counter()
        for k in range(k2):
            L.lopt_set_timing_events(opt.handle, [e.cuda_event for e in ev2[k]])
            opt.step(grads)
        torch.cuda.synchronize()
        ms2 = (time.perf_counter() - t2) * 1e3 / k2
        L.lopt_set_timing_events(opt.handle, [])
        ka = L.KERNEL_NAMES.index("k_apply")
        ap2 = float(np.mean([ev2[k][ka].elapsed_time(ev2[k][ka + 1]) for k in range(k2)]))
        return {"ms_per_step": round(ms2, 4), "value": round(w.n_params / (ms2 * 1e-3) / 1e9, 4),
                "apply_ms": round(ap2, 4), "steps": k2}

    fp32_cmp = other_cmp = None
    other = {L.LOPT_MLP_FP16X3: L.LOPT_MLP_BF16X6, L.LOPT_MLP_BF16X6: L.LOPT_MLP_FP16X3}.get(impl)
    other_name = {L.LOPT_MLP_FP16X3: "fp16x3_path", L.LOPT_MLP_BF16X6: "bf16x6_path"}.get(other)
    if other is not None and not args.no_fp32_compare:
        # the apply kernel switched to the fp32 matrix path, then to the other split path
        log(f"[bench] fp32 matrix path and {other_name} on the same inputs")
        fp32_cmp = time_path(L.LOPT_MLP_MFMA)
        try:
            other_cmp = time_path(other)
        except L.LoptError as err:  # weights outside the fp16x3 path's range
            other_cmp = {"error": str(err)}
    opt.close()
    if args.calibrate_copy:
        src = torch.empty(1 << 28, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)   # reads and writes exactly 1 GiB
        torch.cuda.synchronize()
        del src, dst

    n = w.n_params
    n_vec = sum(t.n for t in w.tensors if t.rows == 1)
    value = n / (ms * 1e-3) / 1e9
    # compulsory bytes of a step: read p, g, m1..3, v and write p, m1..3, v (44 B per element);
    # a 1-D tensor also reads and writes its per-element c1..c3 (68 B)
    step_bytes = 44 * (n - n_vec) + 68 * n_vec
    # algorithmic bytes of the two streaming kernels: g (4 B); g, p, m1..3, v (24 B, 1-D + 12 B)
    stream_bytes = {"k_rowcol_sumsq": 4 * n, "k_stats": 24 * n + 12 * n_vec}
    apply_ms = float(kern_ms[L.KERNEL_NAMES.index("k_apply")])
    fpe = flop_per_elem(args.n_feat)
    fp32_equiv = fpe * n / (apply_ms * 1e-3) / 1e12  # the MLP's fp32 FLOP per second
    use_mfma = impl != L.LOPT_MLP_VALU
    x6 = impl == L.LOPT_MLP_BF16X6
    x3 = impl == L.LOPT_MLP_FP16X3
    # The roofline of the apply kernel is that of the unit its contraction runs
    # on: fp32 matrix cores, the vector ALU, or the fp16 (fp16x3) or bf16
    # (bf16x6) matrix cores, which execute three fp16 or six bf16 piece
    # products per fp32 product.
    if x6:
        achieved, peak, apply_kernel = X6_PRODUCTS * fp32_equiv, PEAK_BF16_MFMA_TFLOPS, "k_apply_bf16x6"
    elif x3:
        achieved, peak, apply_kernel = X3_PRODUCTS * fp32_equiv, PEAK_FP16_MFMA_TFLOPS, "k_apply_fp16x3"
    elif use_mfma:
        achieved, peak, apply_kernel = fp32_equiv, PEAK_FP32_MFMA_TFLOPS, "k_apply_mfma"
    else:
        achieved, peak, apply_kernel = fp32_equiv, PEAK_FP32_VALU_TFLOPS, "k_apply_valu"
    out = {
        "metric": "G params updated/sec per optimizer step; % of HBM / FP32 roofline",
        "value": round(value, 4),
        "unit": "G params/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": (round(value / PAGE_VIT_GPARAMS_PER_S, 3)
                        if w.key == "vit_b16" and args.n_feat == 28 else None),
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"{w.key}: {w.description}", "n_params": n, "n_tensors": len(w.tensors),
                   "mlp_impl": "bf16x6" if x6 else "fp16x3" if x3 else "mfma" if use_mfma else "valu",
                   "state": "zero-init, gradients fixed",
                   "variant": "small_fc_lopt" if args.n_feat == 28 else "VeLO-shaped (19 features, 30 inputs)"},
        "roofline": {"bound": "mfma" if use_mfma else "alu", "kernel": apply_kernel,
                     "achieved": round(achieved, 3), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(achieved / peak, 4),
                     "traffic": committed_traffic(w.key, apply_kernel) if use_mfma and args.n_feat == 28 else None,
                     "flop_per_elem": fpe * (X6_PRODUCTS if x6 else X3_PRODUCTS if x3 else 1), "elems_per_launch": n,
                     "fp32_equivalent": {"achieved": round(fp32_equiv, 3), "peak": PEAK_FP32_MFMA_TFLOPS,
                                         "unit": "TFLOP/s", "frac": round(fp32_equiv / PEAK_FP32_MFMA_TFLOPS, 4)}},
        "step_frac_fp32_peak": round(fpe * n / (ms * 1e-3) / 1e12 / PEAK_FP32_MFMA_TFLOPS, 4),
        "kernels_ms": {name: round(float(t), 4) for name, t in zip(L.KERNEL_NAMES, kern_ms)},
        "fp32_matrix_path": fp32_cmp,
        **({other_name: other_cmp} if other_name else {}),
        "step_ms_median": round(float(np.median(per_step)), 4),
        "step_ms_min": round(float(per_step.min()), 4),
        "step_frac_hbm": round(step_bytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
        "hbm_kernels": {},
    }
    for j, name in enumerate(L.KERNEL_NAMES):
        if name in stream_bytes:
            gbs = stream_bytes[name] / (kern_ms[j] * 1e-3) / 1e9
            out["hbm_kernels"][name] = {"achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                        "frac": round(gbs / PEAK_HBM_GBS, 4), "bytes": stream_bytes[name]}
    if args.peaks:
        import subprocess
        exe = os.path.join(ROOT, "learned_optimizer_step_amd", "lopt_microbench")
        log("[bench] machine-figure microbenchmark")
        res = subprocess.run([exe], capture_output=True, text=True, timeout=120)
        if res.returncode == 0:
            mp = json.loads(res.stdout)
            out["measured_peaks"] = mp
            # the same kernels against what the microbenchmark sustains on this GPU
            out["frac_of_measured"] = {
                "k_apply_vs_mfma_4waves_2chains": round(achieved / mp["mfma_4waves_2chains_tflops"], 4)
                if use_mfma and not (x6 or x3) else None,
                "k_apply_vs_bf16_mfma_4waves_2chains": round(achieved / mp["bf16_mfma_4waves_2chains_tflops"], 4)
                if x6 else None,
                "k_stats_vs_read_bw": round(out["hbm_kernels"]["k_stats"]["achieved"] /
                                            (max(mp["read_bw_TBps"], mp["read_bw_nontemporal_TBps"]) * 1e3), 4),
            }
        else:
            out["measured_peaks"] = {"error": res.stderr[-300:]}
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle on host cores)")
        out["cpu_baseline"] = cpu_baseline()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
