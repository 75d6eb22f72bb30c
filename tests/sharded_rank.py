"""One rank of a row-sharded optimizer step, run as its own process by
tests/test_gpu_sharded.py: binds its shard of every tensor of the test's
workload on cuda:0, steps with the exchanges summed over the ranks by
torch.distributed (gloo, through host copies), and saves its shard's results.

    python sharded_rank.py RANK STEPS OUT.npz     (MASTER_ADDR, MASTER_PORT, WORLD_SIZE in the environment)
"""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402
import torch  # noqa: E402
import torch.distributed as dist  # noqa: E402

from learned_optimizer_step_amd import lopt as L  # noqa: E402
from learned_optimizer_step_amd import workloads as W  # noqa: E402

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
from shard_cases import SHAPES, shard_range, take  # noqa: E402


def main():
    rank, steps, out = int(sys.argv[1]), int(sys.argv[2]), sys.argv[3]
    ranks = int(os.environ["WORLD_SIZE"])
    dist.init_process_group("gloo", rank=rank, world_size=ranks)
    print(f"[rank {rank}] of {ranks}: {steps} steps", flush=True)
    w = W.custom_workload("sharded", SHAPES, grad_std=1e-2, steps=steps, wid=180)
    cut = [shard_range(t, rank, ranks) for t in w.tensors]
    params = [torch.from_numpy(take(W.param_init(w, i), t, *cut[i])).cuda() for i, t in enumerate(w.tensors)]
    opt = L.LOpt(params, W.mlp_weights(11, bias_std=0.1), L.config_from(),
                 global_dims=[(t.rows, t.cols) for t in w.tensors])
    exchange = L.allreduce_through_host()
    for s in range(1, steps + 1):
        grads = [torch.from_numpy(take(W.grad_at(w, i, s), t, *cut[i])).cuda() for i, t in enumerate(w.tensors)]
        opt.step_sharded(grads, exchange)
    torch.cuda.synchronize()
    res = {}
    for i in range(len(params)):
        v = opt.state_views(i)
        res[f"p{i}"] = params[i].cpu().numpy().reshape(v["v"].shape)
        for k in ("m", "v", "r", "c"):
            res[f"{k}{i}"] = v[k].cpu().numpy()
    assert opt.t == steps
    opt.close()
    np.savez(out, **res)
    dist.barrier()
    dist.destroy_process_group()
    print(f"[rank {rank}] done", flush=True)


if __name__ == "__main__":
    main()
