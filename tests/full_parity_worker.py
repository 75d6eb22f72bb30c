"""Computes the oracle's results for the full-size workloads, one file per tensor.

    python tests/full_parity_worker.py OUTDIR [WORKLOAD:STEPS ...]

Started by conftest.py at the beginning of a GPU test run, before any test
touches the device; this process never touches it either (no torch), so its
pool of processes is forked from a CPU-only process.  Writes
OUTDIR/<workload>/<tensor>.npz and then OUTDIR/<workload>/DONE (or FAILED with
the error), workloads in the order given.  Exits when its parent process is
gone.  Test infrastructure: it runs the oracle.
"""
from __future__ import annotations

import multiprocessing as mp
import os
import sys
import traceback

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
for p in (ROOT, HERE):
    if p not in sys.path:
        sys.path.insert(0, p)

import numpy as np  # noqa: E402

import full_parity as FP  # noqa: E402
import oracle  # noqa: E402
from learned_optimizer_step_amd import workloads as W  # noqa: E402

_job = {}


def _init(key, steps, outdir):
    from threadpoolctl import threadpool_limits
    threadpool_limits(limits=1)
    hp = FP.default_hyper()
    _job.update(w=W.get_workload(key), steps=steps, outdir=outdir, hp=hp,
                mlp=oracle.unpack_mlp(W.mlp_weights(), hp.n_time, hp.n_feat))


def _one(i):
    ref = FP.reference_tensor(_job["w"], i, _job["steps"], _job["hp"], _job["mlp"])
    tmp = os.path.join(_job["outdir"], f"{i}.tmp.npz")
    np.savez(tmp, **ref)
    os.replace(tmp, os.path.join(_job["outdir"], f"{i}.npz"))
    return i


def _on_term(signum, frame):
    raise SystemExit(1)    # unwinds the pool's context manager, which terminates the pool


def main():
    import signal
    signal.signal(signal.SIGTERM, _on_term)
    root = sys.argv[1]
    jobs = [(a.split(":")[0], int(a.split(":")[1])) for a in sys.argv[2:]] or list(FP.WORKLOADS)
    parent = os.getppid()
    ctx = mp.get_context("fork")
    for key, steps in jobs:
        d = FP.result_dir(root, key)
        os.makedirs(d, exist_ok=True)
        try:
            w = W.get_workload(key)
            # largest tensors first, so the pool's last round is short
            order = sorted(range(len(w.tensors)), key=lambda i: -w.tensors[i].n * steps)
            with ctx.Pool(FP.n_workers(), initializer=_init, initargs=(key, steps, d)) as pool:
                for _ in pool.imap_unordered(_one, order, chunksize=1 if len(order) < 1000 else 16):
                    if os.getppid() != parent:      # the test run ended
                        pool.terminate()
                        return
            open(os.path.join(d, "DONE"), "w").close()
            print(f"[full-worker] {key}: {len(order)} tensors done", flush=True)
        except Exception:
            with open(os.path.join(d, "FAILED"), "w") as f:
                f.write(traceback.format_exc())
            raise


if __name__ == "__main__":
    main()
