"""The exchange of a row-sharded step through torch.distributed on the host
(gloo, two processes, CPU tensors): every rank ends with the sum over the
ranks, in place, as lopt_step_shard expects between its phases."""
import os
import socket

import pytest

torch = pytest.importorskip("torch")


def _free_port():
    with socket.socket() as s:
        s.bind(("127.0.0.1", 0))
        return s.getsockname()[1]


def _rank(rank, world, port, q):
    import torch.distributed as dist

    from learned_optimizer_step_amd import lopt as L
    os.environ.update(MASTER_ADDR="127.0.0.1", MASTER_PORT=str(port))
    dist.init_process_group("gloo", rank=rank, world_size=world)
    buf = torch.arange(40, dtype=torch.float32) * (rank + 1)
    view = buf[8:24]             # an exchange buffer is a view into the workspace
    L.allreduce_through_host()(view)
    q.put((rank, buf.tolist()))
    dist.barrier()
    dist.destroy_process_group()


def test_two_ranks_sum_in_place():
    import torch.multiprocessing as mp
    world, port = 2, _free_port()
    ctx = mp.get_context("spawn")
    q = ctx.Queue()
    procs = [ctx.Process(target=_rank, args=(r, world, port, q)) for r in range(world)]
    for p in procs:
        p.start()
    got = dict(q.get(timeout=120) for _ in procs)
    for p in procs:
        p.join(timeout=60)
        assert p.exitcode == 0
    for r in range(world):
        want = [float(i * (r + 1)) for i in range(40)]
        for i in range(8, 24):
            want[i] = float(i * 3)           # 1x + 2x over the two ranks
        assert got[r] == want
