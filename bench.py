"""Throughput of the small_fc_lopt optimizer step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload vit_b16]

A step is one lopt_step over the whole parameter list (row/column sums,
moving averages, statistics, finalize, apply).  Inputs (parameters, state,
gradients) are resident in HBM before the timed region; the same gradients
are reused for every timed step.  Prints one JSON line.

The headline is the MLP path that LOPT_MLP_AUTO resolves to (bf16x8: fp32
products from bf16 pieces, each within 2^-30 of itself, fp32 accumulation).  The default run then
times the other matrix paths on the same inputs, each from the same initial
state (parameters, accumulators and step counter restored first): the other
fp32 paths (the fp32 matrix cores, bf16x9 with all nine exact products) and
the two narrower split paths (bf16x6, fp16x3), labelled with their
arithmetic.
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
PEAK_HBM_GBS = 8000.0
# ViT-B/16 step of small_fc_lopt with the fused CUDA kernels on the PyLO page
# ("Benchmark results" > step-time table): 99.59 ms for 86,563,584 parameters.
PAGE_VIT_GPARAMS_PER_S = 86_563_584 / 99.59e-3 / 1e9

# MLP paths: name -> (apply kernel, unit its contraction runs on, unit peak
# TFLOP/s, piece products per fp32 product, arithmetic of the products)
PATHS = {
    "bf16x8": ("k_apply_bf16x8", "bf16 matrix cores", PEAK_BF16_MFMA_TFLOPS, 8,
               "fp32: every product within 2^-30 of itself (eight of the nine bf16 piece products of exact "
               "three-piece splits), fp32 accumulation"),
    "bf16x9": ("k_apply_bf16x9", "bf16 matrix cores", PEAK_BF16_MFMA_TFLOPS, 9,
               "fp32: every product exact (nine bf16 piece products of exact three-piece splits), fp32 accumulation"),
    "mfma": ("k_apply_mfma", "fp32 matrix cores", PEAK_FP32_MFMA_TFLOPS, 1, "fp32"),
    "bf16x6": ("k_apply_bf16x6", "bf16 matrix cores", PEAK_BF16_MFMA_TFLOPS, 6,
               "narrower than fp32: six of the nine bf16 piece products (dropped terms < 2^-21 of each product)"),
    "fp16x3": ("k_apply_fp16x3", "fp16 matrix cores", PEAK_FP16_MFMA_TFLOPS, 3,
               "narrower than fp32: 22-bit operands (two fp16 pieces), three piece products"),
    "valu": ("k_apply_valu", "vector ALU", PEAK_FP32_VALU_TFLOPS, 1, "fp32"),
}


def log(msg):
    print(msg, file=sys.stderr, flush=True)


# Sources of the apply kernel; the committed HBM-traffic figure is only valid
# for the code it was measured on (comments and blank lines do not count).
APPLY_SOURCES = ("learned_optimizer_step_amd/csrc/lopt_apply.hip", "learned_optimizer_step_amd/csrc/lopt_apply_body.h",
                 "learned_optimizer_step_amd/csrc/lopt_device.h", "learned_optimizer_step_amd/csrc/lopt_internal.h")


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


def committed_traffic(workload: str, kernel: str):
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
    from threadpoolctl import threadpool_limits

    import oracle
    from learned_optimizer_step_amd import workloads as W

    cores = len(os.sched_getaffinity(0))
    threads = min(cores, 16)     # BLAS threads: at most 16, a one-GPU host share of cores
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
    return {"value": n / dt / 1e9, "unit": "G params/s", "cores": cores, "threads": threads, "kind": "oracle",
            "sample": f"ViT-B/16 blocks 0-{blocks - 1} ({len(idx)} tensors, {n} params), 1 step, fp64 NumPy "
                      f"(BLAS matmuls on {threads} threads, element-wise work on one), {dt:.1f} s, "
                      f"{cores} host cores visible"}


def roofline(name: str, n: int, n_vec: int, apply_ms: float, fpe: int, traffic, single: bool = False):
    """The apply kernel against the peak of the unit its contraction runs on.

    achieved = algorithmic FLOP (fpe per element: the MLP's fp32 multiply-adds,
    not the piece products a split path issues) over the kernel's time.  A
    one-launch step (single) has no separate apply kernel: its one kernel,
    all five passes, takes that place."""
    kernel, unit, peak, pieces, _ = PATHS[name]
    if single:
        kernel = f"k_step_single ({kernel[len('k_apply_'):]}; all five passes)"
    tflops = fpe * n / (apply_ms * 1e-3) / 1e12
    out = {"bound": "alu" if name == "valu" else "mfma", "kernel": kernel, "unit_of_contraction": unit,
           "achieved": round(tflops, 3), "peak": peak, "unit": "TFLOP/s", "frac": round(tflops / peak, 4),
           "traffic": traffic, "flop_per_elem": fpe, "elems_per_launch": n}
    # compulsory bytes of the apply kernel: read p, g, m1..3, v, write p, m1..3, v
    # (44 B per element; a 1-D tensor also reads and writes its per-element c1..c3: 68 B)
    apply_bytes = 44 * (n - n_vec) + 68 * n_vec
    gbs = apply_bytes / (apply_ms * 1e-3) / 1e9
    out["hbm"] = {"achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                  "bytes": apply_bytes}
    if pieces > 1:
        # share of the unit's peak that the issued piece products use
        out["piece_products"] = pieces
        out["piece_frac"] = round(pieces * tflops / peak, 4)
        fp32_frac = tflops / PEAK_FP32_MFMA_TFLOPS
        if fp32_frac < 1.0:
            out["fp32_equivalent_frac"] = round(fp32_frac, 4)
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="vit_b16")
    ap.add_argument("--impl", default="auto", choices=["auto"] + list(PATHS))
    ap.add_argument("--launch", default="auto", choices=["auto", "split", "single"],
                    help="five kernels per step (split), one (single), or the library's choice (auto: "
                         "split)")
    ap.add_argument("--n-feat", type=int, default=28, choices=(28, 19),
                    help="per-element features: 28 (small_fc_lopt) or 19 (the VeLO-shaped variant)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-fp32-compare", action="store_true",
                    help="skip timing the other matrix paths on the same inputs")
    ap.add_argument("--graph", action="store_true",
                    help="also time the step replayed from a captured HIP graph (default for lists "
                         "under 10 M parameters, where launch latency dominates)")
    ap.add_argument("--peaks", action="store_true",
                    help="also run the machine-figure microbenchmark and include it as measured_peaks")
    ap.add_argument("--shard-of", type=int, default=1,
                    help="time rank 0's share of a row-sharded step over this many ranks: its rows of every "
                         "matrix and its elements of every 1-D tensor, the three phases of lopt_step_shard "
                         "(the exchanges between them need other GPUs and are not made)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="after the timed steps, run one plain 1 GiB device copy (reference for HBM counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); for one rank's share of a "
              f"row-sharded step across W GPUs use --shard-of W", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from learned_optimizer_step_amd import lopt as L
    from learned_optimizer_step_amd import workloads as W

    impl_of = {"auto": L.LOPT_MLP_AUTO, "valu": L.LOPT_MLP_VALU, "mfma": L.LOPT_MLP_MFMA,
               "bf16x6": L.LOPT_MLP_BF16X6, "fp16x3": L.LOPT_MLP_FP16X3, "bf16x9": L.LOPT_MLP_BF16X9,
               "bf16x8": L.LOPT_MLP_BF16X8}
    name_of = {v: k for k, v in impl_of.items() if k != "auto"}
    launch_of = {"auto": L.LOPT_LAUNCH_AUTO, "split": L.LOPT_LAUNCH_SPLIT, "single": L.LOPT_LAUNCH_SINGLE}
    launch_name = {L.LOPT_LAUNCH_SPLIT: "split", L.LOPT_LAUNCH_SINGLE: "single"}
    w = W.get_workload(args.workload)
    log(f"[bench] {w.key}: {len(w.tensors)} tensors, {w.n_params} params; generating inputs")
    dev = torch.device("cuda:0")
    ranks = max(1, args.shard_of)

    def shard(x, t):
        """Rank 0's rows (matrix) or elements (1-D tensor) of t's values."""
        x = x.reshape(t.rows, t.cols)
        if t.rows > 1:
            return np.ascontiguousarray(x[:max(1, t.rows // ranks)])
        return np.ascontiguousarray(x[:, :max(1, t.cols // ranks)])

    params, grads = [], []
    for i, t in enumerate(w.tensors):
        if ranks > 1:
            params.append(torch.from_numpy(shard(W.param_init(w, i), t)).to(dev))
            grads.append(torch.from_numpy(shard(W.grad_at(w, i, 1), t)).to(dev))
        else:
            params.append(torch.from_numpy(W.param_init(w, i).reshape(t.shape)).to(dev))
            grads.append(torch.from_numpy(W.grad_at(w, i, 1).reshape(t.shape)).to(dev))
    mlp = W.mlp_weights(n_feat=args.n_feat)
    opt = L.LOpt(params, mlp, L.config_from(mlp_impl=impl_of[args.impl], n_feat=args.n_feat,
                                            launch=launch_of[args.launch]),
                 global_dims=[(t.rows, t.cols) for t in w.tensors] if ranks > 1 else None)
    if ranks > 1 and w.prewarm_std is not None:
        raise SystemExit("--shard-of takes workloads with zero initial state")
    exchange_floats = [int(b.numel()) for b in opt.shard_sums()] if ranks > 1 else None

    def one_step():
        if ranks > 1:
            opt.step_sharded(grads, lambda buf: None)   # one GPU: no other ranks to exchange with
        else:
            opt.step(grads)
    if w.prewarm_std is not None:
        for i in range(len(w.tensors)):
            st = W.state_init(w, i)
            v = opt.state_views(i)
            for k in ("m", "v", "r", "c"):
                v[k].copy_(torch.from_numpy(st[k]))
    head = name_of[L.lopt_get_mlp_impl(opt.handle)]   # "auto" resolved
    launch = launch_name[L.lopt_get_launch(opt.handle)] if ranks == 1 else "row shard"
    # the initial state, restored before each path is timed
    p0 = [p.clone() for p in params]
    s0 = [s.clone() for s in opt.states]
    torch.cuda.synchronize()

    def restore(path: str, mode: str):
        for p, q in zip(params, p0):
            p.copy_(q)
        for s, q in zip(opt.states, s0):
            s.copy_(q)
        L.lopt_set_config(opt.handle, L.config_from(mlp_impl=impl_of[path], n_feat=args.n_feat,
                                                    launch=launch_of.get(mode, L.LOPT_LAUNCH_AUTO)))
        opt.t = 0    # waits for the device, then resets the step counter

    nk = L.LOPT_N_KERNELS
    stream = torch.cuda.current_stream(dev)

    def time_path(path: str, steps: int, warmup: int, mode: str):
        """warmup untimed steps, then exactly ``steps`` timed ones, from the initial state.
        A one-launch step records its first five events before its kernel, so
        its whole time counts as k_apply's."""
        restore(path, mode)
        for _ in range(warmup):
            one_step()
        events = [[torch.cuda.Event(enable_timing=True) for _ in range(nk + 1)] for _ in range(steps)]
        for evs in events:          # torch creates the HIP event on first record
            for e in evs:
                e.record(stream)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for k in range(steps):
            L.lopt_set_timing_events(opt.handle, [e.cuda_event for e in events[k]])
            one_step()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        L.lopt_set_timing_events(opt.handle, [])
        kern = np.array([[events[k][j].elapsed_time(events[k][j + 1]) for j in range(nk)] for k in range(steps)])
        per_step = np.array([events[k][0].elapsed_time(events[k][nk]) for k in range(steps)])
        return (t1 - t0) * 1e3 / steps, kern.mean(axis=0), per_step

    log(f"[bench] {head}, {launch} launch: warmup {args.warmup} steps, then {args.steps} timed")
    ms, kern_ms, per_step = time_path(head, args.steps, args.warmup, launch)

    def time_graph(mode: str):
        """One step captured into a HIP graph and replayed: the step's kernels
        without the host's per-launch work (the step counter lives on the
        device, so replays see t = 1, 2, ...)."""
        restore(head, mode)
        opt.step(grads)                    # binds the gradient pointers outside the capture
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            opt.step(grads)
        for _ in range(args.warmup):
            g.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            g.replay()
        torch.cuda.synchronize()
        gms = (time.perf_counter() - t0) * 1e3 / args.steps
        del g
        return {"ms_per_step": round(gms, 4), "value": round(w.n_params / (gms * 1e-3) / 1e9, 4),
                "steps": args.steps, "launches_per_step": 1 if mode == "single" else nk}

    graph, launches = None, None
    if ranks == 1 and (args.graph or w.n_params < 10_000_000):
        log("[bench] graph replay")
        graph = time_graph(launch)
        # the other launch mode, eager and replayed, on the same inputs and initial state
        other = "split" if launch == "single" else "single"
        log(f"[bench] {other} launch, eager and graph replay")
        ms_o, _, _ = time_path(head, args.steps, args.warmup, other)
        launches = {launch: {"ms_per_step": round(ms, 4), "value": round(w.n_params / (ms * 1e-3) / 1e9, 4),
                             "launches_per_step": 1 if launch == "single" else nk, "graph_replay": graph},
                    other: {"ms_per_step": round(ms_o, 4), "value": round(w.n_params / (ms_o * 1e-3) / 1e9, 4),
                            "launches_per_step": 1 if other == "single" else nk, "graph_replay": time_graph(other)}}

    fpe = flop_per_elem(args.n_feat)
    n = sum(int(p.numel()) for p in params)                 # the whole list, or rank 0's share of it
    n_vec = sum(int(p.numel()) for p, t in zip(params, w.tensors) if t.rows == 1)

    side_paths = {}
    if not args.no_fp32_compare:
        others = [p for p in ("mfma", "bf16x8", "bf16x9", "bf16x6", "fp16x3") if p != head]
        log(f"[bench] the same inputs and initial state on {', '.join(others)}")
        for p in others:
            try:
                ms2, k2, _ = time_path(p, 20, 2, launch)
            except L.LoptError as err:  # weights outside the fp16x3 path's range
                side_paths[p] = {"error": str(err)}
                continue
            ap2 = float(k2[L.KERNEL_NAMES.index("k_apply")])
            side_paths[p] = {"ms_per_step": round(ms2, 4), "value": round(n / (ms2 * 1e-3) / 1e9, 4),
                             "apply_ms": round(ap2, 4), "steps": 20, "arithmetic": PATHS[p][4],
                             "apply_frac_of_unit_peak": round(fpe * n / (ap2 * 1e-3) / 1e12 / PATHS[p][2], 4)}
    opt.close()
    if args.calibrate_copy:
        src = torch.empty(1 << 28, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)   # reads and writes exactly 1 GiB
        torch.cuda.synchronize()
        del src, dst

    value = n / (ms * 1e-3) / 1e9
    # compulsory bytes of a step: read p, g, m1..3, v and write p, m1..3, v (44 B per element);
    # a 1-D tensor also reads and writes its per-element c1..c3 (68 B)
    step_bytes = 44 * (n - n_vec) + 68 * n_vec
    # algorithmic bytes of the two streaming kernels: g (4 B); g, p, m1..3, v (24 B, 1-D + 12 B)
    stream_bytes = {"k_rowcol_sumsq": 4 * n, "k_stats": 24 * n + 12 * n_vec}
    apply_ms = float(kern_ms[L.KERNEL_NAMES.index("k_apply")])
    kernel = PATHS[head][0]
    traffic = committed_traffic(w.key, kernel) if args.n_feat == 28 else None
    step_fp32 = fpe * n / (ms * 1e-3) / 1e12 / PEAK_FP32_MFMA_TFLOPS
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
                        if w.key == "vit_b16" and args.n_feat == 28 and ranks == 1 else None),
        "dtype": "f32" if head in ("bf16x8", "bf16x9", "mfma", "valu") else head,
        "data": "synthetic",
        "config": {"workload": f"{w.key}: {w.description}" + (f"; rank 0 of {ranks} row shards" if ranks > 1 else ""),
                   "n_params": n, "n_tensors": len(w.tensors),
                   "mlp_impl": head, "mlp_arithmetic": PATHS[head][4], "launch": launch,
                   "state": "zero-init, gradients fixed" if w.prewarm_std is None else "pre-warmed, gradients fixed",
                   "variant": "small_fc_lopt" if args.n_feat == 28 else "VeLO-shaped (19 features, 30 inputs)"},
        "roofline": roofline(head, n, n_vec, apply_ms, fpe, traffic if launch == "split" else None,
                             single=launch == "single"),
        "kernels_ms": {name: round(float(t), 4) for name, t in zip(L.KERNEL_NAMES, kern_ms)},
        "step_ms_median": round(float(np.median(per_step)), 4),
        "step_ms_min": round(float(per_step.min()), 4),
        "step_frac_hbm": round(step_bytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
        "hbm_kernels": {},
    }
    if step_fp32 < 1.0:
        # the whole step's MLP work over the fp32 matrix peak
        out["step_frac_fp32_peak"] = round(step_fp32, 4)
    if graph is not None:
        out["graph_replay"] = graph
        out["launch_modes"] = launches
    if ranks > 1:
        out["row_shards"] = {"ranks": ranks, "rank": 0, "whole_list_params": w.n_params,
                             "exchange_floats": exchange_floats,
                             "exchange_note": "the two in-place sums over the ranks between the phases are not "
                                              "made on one GPU; the events around the finalize include the gap"}
    out["other_paths"] = side_paths
    for j, name in enumerate(L.KERNEL_NAMES):
        if name in stream_bytes and launch == "split":
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
            achieved = out["roofline"]["achieved"]
            out["frac_of_measured"] = {
                "k_apply_vs_mfma_4waves_2chains": round(achieved / mp["mfma_4waves_2chains_tflops"], 4)
                if head == "mfma" else None,
                "k_stats_vs_read_bw": round(out["hbm_kernels"]["k_stats"]["achieved"] /
                                            (max(mp["read_bw_TBps"], mp["read_bw_nontemporal_TBps"]) * 1e3), 4)
                if "k_stats" in out["hbm_kernels"] else None,
            }
        else:
            out["measured_peaks"] = {"error": res.stderr[-300:]}
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle on host cores)")
        out["cpu_baseline"] = cpu_baseline()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
