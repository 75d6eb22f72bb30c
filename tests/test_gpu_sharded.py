"""Row-shard bindings (lopt_init_state_sharded, lopt_step_shard) on one GPU.

Each whole tensor is cut into shards (a 2-D tensor by rows, a 1-D tensor by
elements) that separate optimizers bind, as the ranks of a sharded step
would; between the phases of a step the exchange buffers are summed over the
shards, as an all-reduce across ranks would.  The shards' results, put back
together, must equal the oracle's step of the whole tensors to the parity
bar; with one shard the three phases must equal lopt_step bit for bit.  A
two-process run exchanges through torch.distributed (gloo, host copies).
"""
import os
import socket
import subprocess
import sys

import numpy as np
import pytest

from gpu_harness import compare, compare_stats, hyper_from_cfg, oracle_run, say
from shard_cases import SHAPES, shard_range, take

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("no GPU", allow_module_level=True)

from learned_optimizer_step_amd import lopt as L  # noqa: E402
from learned_optimizer_step_amd import workloads as W  # noqa: E402

class Shards:
    """The shards of workload w on one GPU, one optimizer per rank."""

    def __init__(self, w, ranks, cfg, mlp):
        self.w, self.ranks = w, ranks
        dims = [(t.rows, t.cols) for t in w.tensors]
        self.cut = [[shard_range(t, k, ranks) for t in w.tensors] for k in range(ranks)]
        self.opts, self.params = [], []
        for k in range(ranks):
            ps = [torch.from_numpy(take(W.param_init(w, i), t, *self.cut[k][i])).cuda()
                  for i, t in enumerate(w.tensors)]
            self.params.append(ps)
            self.opts.append(L.LOpt(ps, mlp, cfg, global_dims=dims))

    def step(self, t, skip=()):
        """Step t; the tensors in skip have no gradient in it (on every shard)."""
        grads = [[None if i in skip else torch.from_numpy(take(W.grad_at(self.w, i, t), tt, *self.cut[k][i])).cuda()
                  for i, tt in enumerate(self.w.tensors)] for k in range(self.ranks)]
        sums = [o.shard_sums() for o in self.opts]
        for phase in range(3):
            for k, o in enumerate(self.opts):
                o.step_shard_phase(phase, grads[k] if phase == 0 else None)
            if phase < 2:   # the exchange: every shard gets the sum over the shards
                total = sum(s[phase] for s in sums)
                for s in sums:
                    s[phase].copy_(total)

    def gather(self, i):
        """Tensor i put back together: p, m, v, r, c as the oracle holds them."""
        t = self.w.tensors[i]
        views = [o.state_views(i) for o in self.opts]
        if t.rows > 1:
            out = {"p": np.concatenate([p[i].cpu().numpy().reshape(-1, t.cols) for p in self.params]),
                   "m": np.concatenate([v["m"].cpu().numpy() for v in views], axis=1),
                   "v": np.concatenate([v["v"].cpu().numpy() for v in views], axis=0),
                   "r": np.concatenate([v["r"].cpu().numpy() for v in views], axis=1),
                   "c": views[0]["c"].cpu().numpy()}
            for v in views[1:]:   # every shard holds the same column accumulators
                assert np.array_equal(v["c"].cpu().numpy(), out["c"]), f"tensor {i}: shards' c differ"
        else:
            out = {"p": np.concatenate([p[i].cpu().numpy().reshape(1, -1) for p in self.params], axis=1),
                   "m": np.concatenate([v["m"].cpu().numpy() for v in views], axis=2),
                   "v": np.concatenate([v["v"].cpu().numpy() for v in views], axis=1),
                   "r": views[0]["r"].cpu().numpy(),
                   "c": np.concatenate([v["c"].cpu().numpy() for v in views], axis=1)}
            for v in views[1:]:   # a 1-D tensor's r_k is one value, the same on every shard
                assert np.array_equal(v["r"].cpu().numpy(), out["r"]), f"tensor {i}: shards' r differ"
        return out

    def close(self):
        for o in self.opts:
            o.close()


@pytest.mark.parametrize("ranks", [2, 3])
@pytest.mark.parametrize("impl,n_feat", [(L.LOPT_MLP_AUTO, 28), (L.LOPT_MLP_MFMA, 28), (L.LOPT_MLP_AUTO, 19)])
def test_shards_equal_the_oracle_on_the_whole_tensors(ranks, impl, n_feat):
    steps = 4
    w = W.custom_workload("sharded", SHAPES, grad_std=1e-2, steps=steps, wid=180)
    cfg = L.config_from(mlp_impl=impl, n_feat=n_feat)
    mlp = W.mlp_weights(11, bias_std=0.1, n_feat=n_feat)
    say(f"[sharded] {ranks} shards, impl {impl}, n_feat {n_feat}")
    sh = Shards(w, ranks, cfg, mlp)
    for t in range(1, steps + 1):
        sh.step(t)
    torch.cuda.synchronize()
    want = oracle_run(w, mlp, hyper_from_cfg(cfg), steps)
    errs = []
    for i, t in enumerate(w.tensors):
        label = f"shards[{i}:{t.rows}x{t.cols}]"
        errs += compare(sh.gather(i), want[i], label)
        for k, o in enumerate(sh.opts):   # every shard normalised with the whole tensor's statistics
            errs += compare_stats(o.tensor_stats()[i], want[i], n_feat, f"{label} shard {k}")
    assert all(o.t == steps for o in sh.opts)
    sh.close()
    assert not errs, "\n".join(errs[:20])


def test_shards_with_per_tensor_values_and_skipped_gradients():
    """Per-tensor learning rates and weight decays (the same on every shard),
    and a tensor without a gradient in one step, against the oracle with the
    same values and the same skip."""
    steps = 4
    w = W.custom_workload("sharded", SHAPES, grad_std=1e-2, steps=steps, wid=180)
    cfg = L.config_from()
    mlp = W.mlp_weights(11, bias_std=0.1)
    th = [(0.5 + 0.1 * i, 0.01 * (i % 3)) for i in range(len(SHAPES))]
    sh = Shards(w, 2, cfg, mlp)
    for o in sh.opts:
        o.set_tensor_hyper([a for a, _ in th], [b for _, b in th])
    skip_step, skipped = 3, 4
    for t in range(1, steps + 1):
        sh.step(t, skip=(skipped,) if t == skip_step else ())
    torch.cuda.synchronize()
    # the oracle: tensor `skipped` takes steps 1, 2 and 4 (t still counts 1, 2, 4), the others all four
    want = oracle_run(w, mlp, hyper_from_cfg(cfg), steps, tensor_hyper=th)
    errs = []
    for i, t in enumerate(w.tensors):
        if i == skipped:
            continue
        errs += compare(sh.gather(i), want[i], f"per-tensor[{i}]")
    import dataclasses
    import oracle
    hp = dataclasses.replace(hyper_from_cfg(cfg).as_f32(), lr=float(np.float32(th[skipped][0])),
                             weight_decay=float(np.float32(th[skipped][1])))
    m = oracle.unpack_mlp(mlp, hp.n_time, hp.n_feat)
    p, st = W.param_init(w, skipped), W.state_init(w, skipped)
    for t in (1, 2, 4):
        p, st, _ = oracle.step_tensor(p, W.grad_at(w, skipped, t), st, t, m, hp)
    errs += compare(sh.gather(skipped), dict(p=p, **st), f"skipped[{skipped}]")
    sh.close()
    assert not errs, "\n".join(errs[:20])


@pytest.mark.parametrize("impl", [L.LOPT_MLP_AUTO, L.LOPT_MLP_MFMA])
def test_one_shard_is_lopt_step_bit_for_bit(impl):
    w = W.custom_workload("sharded_one", SHAPES + [(1, 1)], grad_std=1e-2, steps=5, wid=181)
    mlp = W.mlp_weights(11, bias_std=0.1)
    cfg = L.config_from(mlp_impl=impl)
    pa = [torch.from_numpy(W.param_init(w, i).reshape(t.shape)).cuda() for i, t in enumerate(w.tensors)]
    pb = [p.clone() for p in pa]
    a = L.LOpt(pa, mlp, cfg, global_dims=[(t.rows, t.cols) for t in w.tensors])
    b = L.LOpt(pb, mlp, cfg)
    for s in range(1, 6):
        g = [torch.from_numpy(W.grad_at(w, i, s).reshape(t.shape)).cuda() for i, t in enumerate(w.tensors)]
        if s == 3:
            g[1] = None   # a tensor without a gradient in one step
        a.step_sharded(g, lambda buf: None)
        b.step(g)
    torch.cuda.synchronize()
    for i in range(len(pa)):
        assert torch.equal(pa[i], pb[i]), i
        assert torch.equal(a.states[i], b.states[i]), i
    assert np.array_equal(a.tensor_stats(), b.tensor_stats())
    assert a.t == b.t == 5
    a.close()
    b.close()


def test_phase_order_and_plain_step_are_refused():
    p = torch.zeros(8, 8, device="cuda")
    o = L.LOpt([p], W.mlp_weights(), L.config_from(), global_dims=[(16, 8)])
    g = [torch.full((8, 8), 1e-3, device="cuda")]
    with pytest.raises(L.LoptError):
        o.step(g)
    with pytest.raises(L.LoptError):
        o.step_shard_phase(1)
    o.step_shard_phase(0, g)
    with pytest.raises(L.LoptError):
        o.step_shard_phase(0, g)
    o.step_shard_phase(1)
    o.step_shard_phase(2)
    assert o.t == 1
    s1, s2 = o.shard_sums()
    assert s1.numel() == 8 and s2.numel() == 32
    o.close()


def free_port():
    with socket.socket() as s:
        s.bind(("127.0.0.1", 0))
        return s.getsockname()[1]


def test_two_processes_exchange_through_torch_distributed(tmp_path):
    """Two ranks in two processes on the one GPU, the exchange an all-reduce
    of torch.distributed (gloo, through host copies)."""
    ranks, steps = 2, 3
    port = str(free_port())
    script = os.path.join(os.path.dirname(os.path.abspath(__file__)), "sharded_rank.py")
    env = dict(os.environ, MASTER_ADDR="127.0.0.1", MASTER_PORT=port, WORLD_SIZE=str(ranks))
    procs = [subprocess.Popen([sys.executable, "-u", script, str(k), str(steps), str(tmp_path / f"rank{k}.npz")],
                              env=dict(env, RANK=str(k)), stdout=subprocess.PIPE, stderr=subprocess.STDOUT)
             for k in range(ranks)]
    outs = []
    for p in procs:
        try:
            out, _ = p.communicate(timeout=240)
        except subprocess.TimeoutExpired:
            for q in procs:
                q.kill()
            raise
        outs.append(out.decode(errors="replace"))
        assert p.returncode == 0, outs[-1][-3000:]
    w = W.custom_workload("sharded", SHAPES, grad_std=1e-2, steps=steps, wid=180)
    cfg = L.config_from()
    mlp = W.mlp_weights(11, bias_std=0.1)
    want = oracle_run(w, mlp, hyper_from_cfg(cfg), steps)
    parts = [np.load(tmp_path / f"rank{k}.npz") for k in range(ranks)]
    errs = []
    for i, t in enumerate(w.tensors):
        if t.rows > 1:
            got = {"p": np.concatenate([q[f"p{i}"] for q in parts]),
                   "m": np.concatenate([q[f"m{i}"] for q in parts], axis=1),
                   "v": np.concatenate([q[f"v{i}"] for q in parts], axis=0),
                   "r": np.concatenate([q[f"r{i}"] for q in parts], axis=1), "c": parts[0][f"c{i}"]}
        else:
            got = {"p": np.concatenate([q[f"p{i}"] for q in parts], axis=1),
                   "m": np.concatenate([q[f"m{i}"] for q in parts], axis=2),
                   "v": np.concatenate([q[f"v{i}"] for q in parts], axis=1),
                   "r": parts[0][f"r{i}"], "c": np.concatenate([q[f"c{i}"] for q in parts], axis=1)}
        errs += compare(got, want[i], f"two processes[{i}]")
    assert not errs, "\n".join(errs[:20])
