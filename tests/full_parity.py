"""Parity on the full-size workloads: every tensor of the list, on every MLP path.

The oracle's results for these workloads are computed once, in a separate
worker process (tests/full_parity_worker.py) that conftest.py starts when a GPU
run begins, before any test touches the device: it steps the tensors on a pool
of processes while the other GPU tests run, and writes one file per tensor.
The tests here load them and compare each MLP path's GPU step against them;
the inputs are generated once per workload (threads: NumPy's generator
releases the interpreter lock) and stay on the device between the paths.
Without the worker (a single test file run on its own) the reference is
computed in this process instead.

Per tensor, element by element to the parity bar:
* r_k and c_k (every row and column) and the statistics of the step (the
  feature normalisers s_d and sqrt(mean r_k), lopt_get_tensor_stats); a 1-D
  tensor's c_k is per element and is compared where its p, m, v are;
* p, m_a and v everywhere for a tensor of at most CAP elements (the 4096 x
  4096 weight: everywhere); above it at >= 16 sampled rows, first and last
  included (a 1-D tensor: >= 16 windows of 1024 elements, first and last
  included).  The oracle computes every per-tensor sum over the whole tensor
  either way (step_tensor_sub);
* a workload of several steps is followed in full (each step's features read
  every element's parameters), so p, m, v are compared everywhere.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import time
from typing import Dict, List, Optional

import numpy as np

import oracle
from learned_optimizer_step_amd import workloads as W

RTOL = 1e-5            # the parity bar (as in gpu_harness)
ATOL = 1e-7
CAP = 1 << 16          # elements compared everywhere up to this size
N_ROWS = 16            # sampled rows (or 1-D windows) above it, plus the first and last
WINDOW = 1024          # elements per sampled 1-D window

# (workload, steps): each workload's own step count (reading R20)
WORKLOADS = (("single4096", 1), ("vit_b16", 5), ("gpt2_355m", 1), ("llama1b", 1), ("ragged10k", 1))
# workloads whose every element is compared whatever the tensor size
EVERYWHERE = ("single4096",)


def say(msg: str) -> None:
    print(msg, flush=True)


def n_workers() -> int:
    """The host cores this process may use, at most 16 (a one-GPU host share)."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def sample_of(w: W.Workload, i: int, steps: int):
    """(rows, cols) compared for tensor i of w, None meaning all."""
    t = w.tensors[i]
    if t.n <= CAP or steps > 1 or w.key in EVERYWHERE:
        return None, None
    rng = np.random.default_rng(1000 + i)
    if t.rows > 1:
        rows = sorted(set([0, t.rows - 1] + rng.choice(t.rows, min(t.rows, N_ROWS), replace=False).tolist()))
        return rows, None
    starts = set([0, t.cols - WINDOW] + rng.integers(0, t.cols - WINDOW, N_ROWS).tolist())
    return None, np.unique(np.concatenate([np.arange(s, s + WINDOW) for s in sorted(starts)])).tolist()


def default_hyper() -> oracle.Hyper:
    """The library's default configuration (lopt_default_config), as the oracle's fp32 numbers."""
    return oracle.Hyper().as_f32()


def reference_tensor(w: W.Workload, i: int, steps: int, hp: oracle.Hyper, mlp: oracle.Mlp) -> Dict[str, np.ndarray]:
    """The oracle's result for tensor i of workload w after ``steps`` steps."""
    p = W.param_init(w, i)
    st = W.state_init(w, i)
    rows, cols = sample_of(w, i, steps)
    if steps == 1:
        pn, sn, info = oracle.step_tensor_sub(p, W.grad_at(w, i, 1), st, 1, mlp, hp, rows, cols)
    else:
        for s in range(1, steps + 1):
            p, st, info = oracle.step_tensor(p, W.grad_at(w, i, s), st, s, mlp, hp)
        pn, sn = oracle.as_matrix(p), st
    rbar = np.asarray(sn["r"], np.float64).mean(axis=1)
    c = sn["c"]
    if cols is not None:     # a 1-D tensor's c_k is per element: compared where p, m, v are
        c = np.asarray(c)[:, cols]
    return dict(p=pn, m=sn["m"], v=sn["v"], r=sn["r"], c=c, scales=np.asarray(info.scales, np.float64),
                sqrt_rbar=np.sqrt(rbar))


def result_dir(root: str, key: str) -> str:
    return os.path.join(root, key)


def load_reference(root: Optional[str], key: str, steps: int, timeout: float = 900.0) -> List[Dict[str, np.ndarray]]:
    """The worker's results for ``key`` (waiting for them), or, without a
    worker, the oracle run here on a pool of threads."""
    w = W.get_workload(key)
    if root is not None:
        d = result_dir(root, key)
        t0 = last = time.time()
        while not os.path.exists(os.path.join(d, "DONE")):
            if os.path.exists(os.path.join(d, "FAILED")):
                raise RuntimeError(open(os.path.join(d, "FAILED")).read())
            now = time.time()
            if now - t0 > timeout:
                raise TimeoutError(f"oracle results for {key} not ready after {timeout:.0f} s")
            if now - last > 30:
                have = len([f for f in os.listdir(d)]) if os.path.isdir(d) else 0
                say(f"[full] {key}: waiting for the oracle worker ({have}/{len(w.tensors)} tensors, {now - t0:.0f} s)")
                last = now
            time.sleep(2.0)
        say(f"[full] {key}: oracle results ready (waited {time.time() - t0:.0f} s)")
        out = []
        for i in range(len(w.tensors)):
            with np.load(os.path.join(d, f"{i}.npz")) as z:
                out.append({k: z[k] for k in z.files})
        return out
    say(f"[full] {key}: no oracle worker; computing the reference here ({n_workers()} threads)")
    hp = default_hyper()
    mlp = oracle.unpack_mlp(W.mlp_weights(), hp.n_time, hp.n_feat)
    from threadpoolctl import threadpool_limits
    with threadpool_limits(limits=1):
        with cf.ThreadPoolExecutor(n_workers()) as ex:
            return list(ex.map(lambda i: reference_tensor(w, i, steps, hp, mlp), range(len(w.tensors))))


class DeviceInputs:
    """A workload's seeded inputs on the device (parameters, each step's
    gradients, pre-warmed state), generated on a pool of threads."""

    def __init__(self, w: W.Workload, steps: int, torch):
        nt = len(w.tensors)

        def gen(i):
            t = w.tensors[i]
            return (torch.from_numpy(W.param_init(w, i).reshape(t.shape)),
                    [torch.from_numpy(W.grad_at(w, i, s).reshape(t.shape)) for s in range(1, steps + 1)],
                    W.state_init(w, i) if w.prewarm_std is not None else None)

        with cf.ThreadPoolExecutor(n_workers()) as ex:
            host = list(ex.map(gen, range(nt)))
        self.p0 = [h[0].cuda() for h in host]
        self.grads = [[h[1][s].cuda() for h in host] for s in range(steps)]
        self.state0 = [h[2] for h in host]
        torch.cuda.synchronize()


def gpu_compare(w: W.Workload, steps: int, want: List[Dict[str, np.ndarray]], dev: DeviceInputs, mlp: np.ndarray,
                cfg, torch) -> List[str]:
    """The GPU's steps on one MLP path against the reference, on every tensor."""
    from gpu_harness import compare, compare_stats
    from learned_optimizer_step_amd import lopt as L

    say(f"[full] {w.key}: GPU, impl={cfg.mlp_impl}")
    params = [p.clone() for p in dev.p0]
    opt = L.LOpt(params, mlp, cfg)
    for i, st in enumerate(dev.state0):
        if st is not None:
            v = opt.state_views(i)
            for k in ("m", "v", "r", "c"):
                v[k].copy_(torch.from_numpy(st[k]))
    for s in range(steps):
        opt.step(dev.grads[s])
    torch.cuda.synchronize()
    stats = opt.tensor_stats()
    # what is compared, gathered on the device, then one copy to the host
    keys = ("p", "m", "v", "r", "c")
    pieces, shapes = [], []
    for i, t in enumerate(w.tensors):
        rows, cols = sample_of(w, i, steps)
        v = opt.state_views(i)
        p, m, vv, cc = params[i].view(t.rows, t.cols), v["m"], v["v"], v["c"]
        if rows is not None:
            ri = torch.tensor(rows, device=p.device)
            p, m, vv = p.index_select(0, ri), m.index_select(1, ri), vv.index_select(0, ri)
        if cols is not None:   # only 1-D tensors sample columns; their c_k is per element
            ci = torch.tensor(cols, device=p.device)
            p, m, vv, cc = p.index_select(1, ci), m.index_select(2, ci), vv.index_select(1, ci), cc.index_select(1, ci)
        for x in (p, m, vv, v["r"], cc):
            pieces.append(x.reshape(-1))
            shapes.append(tuple(x.shape))
    flat = torch.cat(pieces).cpu().numpy()
    opt.close()
    del opt, params, pieces
    errs = []
    off = 0
    nf = int(cfg.n_feat)
    for i, t in enumerate(w.tensors):
        got = {}
        for j, k in enumerate(keys):
            shp = shapes[5 * i + j]
            cnt = int(np.prod(shp))
            got[k] = flat[off:off + cnt].reshape(shp)
            off += cnt
        ref = want[i]
        label = f"{w.key}[{i}:{t.name} {t.rows}x{t.cols}]"
        errs += compare(got, ref, label)
        errs += compare_stats(stats[i], ref, nf, label)
    say(f"[full] {w.key}: impl={cfg.mlp_impl}: {len(w.tensors)} tensors compared, {len(errs)} failures")
    return errs
