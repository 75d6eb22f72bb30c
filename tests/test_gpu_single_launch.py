"""The one-launch step (LOPT_LAUNCH_SINGLE) against the five-kernel step
(LOPT_LAUNCH_SPLIT).

Both run the same per-item bodies in the same order of items within each
pass (the one-launch kernel takes them in a block-stride loop and separates
the passes with grid-wide barriers), so their results must agree bit for bit:
parameters, every accumulator, the per-tensor statistics and the step
counter, on every MLP path.  LOPT_LAUNCH_AUTO runs the five kernels, which
test_gpu_parity.py holds to the oracle; test_one_launch_against_the_oracle
below holds the one-launch step to it directly.
"""
import numpy as np
import pytest

from gpu_harness import IMPLS, compare, oracle_run, hyper_from_cfg, say

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("no GPU", allow_module_level=True)

from learned_optimizer_step_amd import lopt as L  # noqa: E402
from learned_optimizer_step_amd import workloads as W  # noqa: E402

SINGLE, SPLIT, AUTO = L.LOPT_LAUNCH_SINGLE, L.LOPT_LAUNCH_SPLIT, L.LOPT_LAUNCH_AUTO

MIXED = [(1,), (3,), (63,), (65,), (40000,), (1, 1), (2, 3), (17, 33), (4, 513), (129, 257), (1000, 1),
         (2, 64), (64, 64), (7, 4096), (9, 65), (3, 4097), (300, 256)]


def run(w, impl, launch, steps, n_feat=L.LOPT_N_FEATURES, skip=None, tensor_hyper=None, bias_std=0.1, edit=None):
    """Steps ``w`` from its seeded start; skip(t, i) -> True leaves tensor i
    without a gradient in step t; edit(t, i, g) may change gradient i of step
    t (a numpy array) in place.  Returns (params, states, stats, t, launch the
    handle resolved)."""
    cfg = L.config_from(mlp_impl=impl, launch=launch, n_feat=n_feat)
    params = [torch.from_numpy(W.param_init(w, i).reshape(t.shape)).cuda() for i, t in enumerate(w.tensors)]
    opt = L.LOpt(params, W.mlp_weights(11, bias_std=bias_std, n_feat=n_feat), cfg)
    if w.prewarm_std is not None:
        for i in range(len(w.tensors)):
            st = W.state_init(w, i)
            v = opt.state_views(i)
            for k in ("m", "v", "r", "c"):
                v[k].copy_(torch.from_numpy(st[k]))
    if tensor_hyper is not None:
        opt.set_tensor_hyper([a for a, _ in tensor_hyper], [b for _, b in tensor_hyper])
    for t in range(1, steps + 1):
        grads = []
        for i, tt in enumerate(w.tensors):
            if skip is not None and skip(t, i):
                grads.append(None)
                continue
            g = W.grad_at(w, i, t)
            if edit is not None:
                edit(t, i, g)
            grads.append(torch.from_numpy(g.reshape(tt.shape)).cuda())
        opt.step(grads)
    torch.cuda.synchronize()
    mode = L.lopt_get_launch(opt.handle)
    out = ([p.clone() for p in params], [s.clone() for s in opt.states], opt.tensor_stats(), opt.t, mode)
    opt.close()
    return out


def same(x, y):
    """Equal bit for bit, except that a NaN equals any NaN (payloads aside)."""
    nx, ny = torch.isnan(x), torch.isnan(y)
    return torch.equal(nx, ny) and torch.equal(torch.where(nx, 0, x), torch.where(ny, 0, y))


def assert_same(a, b, label):
    pa, sa, sta, ta, _ = a
    pb, sb, stb, tb, _ = b
    assert ta == tb, (label, ta, tb)
    for i in range(len(pa)):
        assert same(pa[i], pb[i]), f"{label}: parameters of tensor {i} differ"
        assert same(sa[i], sb[i]), f"{label}: state of tensor {i} differs"
    assert np.array_equal(sta, stb, equal_nan=True), f"{label}: statistics differ"


@pytest.mark.parametrize("impl", IMPLS)
def test_single256_ten_steps_bitwise(impl):
    w = W.get_workload("single256")
    a = run(w, impl, SINGLE, 10)
    b = run(w, impl, SPLIT, 10)
    assert a[4] == SINGLE and b[4] == SPLIT
    assert_same(a, b, f"single256 impl {impl}")


@pytest.mark.parametrize("impl", IMPLS)
@pytest.mark.parametrize("n_feat", [L.LOPT_N_FEATURES, L.LOPT_VELO_FEATURES])
def test_mixed_shapes_skips_and_per_tensor_values_bitwise(impl, n_feat):
    """1-D, row-uniform and mixed-row matrices, tensors without a gradient in
    some steps, and per-tensor learning rates and weight decays."""
    w = W.custom_workload("single_mixed", MIXED, grad_std=1e-2, steps=6, wid=160)
    th = [(0.5 + 0.1 * i, 0.01 * (i % 3)) for i in range(len(MIXED))]
    skip = lambda t, i: (t + i) % 4 == 0  # noqa: E731
    a = run(w, impl, SINGLE, 6, n_feat=n_feat, skip=skip, tensor_hyper=th)
    b = run(w, impl, SPLIT, 6, n_feat=n_feat, skip=skip, tensor_hyper=th)
    assert_same(a, b, f"mixed impl {impl} n_feat {n_feat}")


def test_auto_takes_five_launches_and_2_20_elements_bitwise():
    w = W.custom_workload("auto_small", [(1024, 1024)], steps=1, wid=161)   # 2^20 elements
    a = run(w, L.LOPT_MLP_AUTO, AUTO, 2)
    assert a[4] == SPLIT
    b = run(w, L.LOPT_MLP_AUTO, SINGLE, 2)
    assert b[4] == SINGLE
    assert_same(a, b, "2^20 elements")


@pytest.mark.parametrize("bad", [float("nan"), float("inf")])
def test_non_finite_gradient_element_as_five_kernels(bad):
    """A NaN or Inf in one gradient element reaches the same accumulators and
    parameters as with the five kernels (the one-launch kernel's streaming
    passes are compiled with -fno-honor-nans)."""
    w = W.custom_workload("single_nonfinite", [(64, 96), (1, 300), (40, 7), (33, 64)], grad_std=1e-2, steps=3, wid=167)

    def edit(t, i, g):
        if t == 2 and i in (0, 1):
            g.reshape(-1)[17] = bad

    a = run(w, L.LOPT_MLP_AUTO, SINGLE, 3, edit=edit)
    b = run(w, L.LOPT_MLP_AUTO, SPLIT, 3, edit=edit)
    assert not torch.isfinite(a[1][0]).all()      # the bad value did reach tensor 0's state
    assert torch.isfinite(a[0][3]).all()          # and stayed out of tensor 3
    assert_same(a, b, f"non-finite {bad}")


@pytest.mark.parametrize("impl", [L.LOPT_MLP_BF16X8, L.LOPT_MLP_MFMA])
def test_vit_b16_forced_one_launch_bitwise(impl):
    """A list far larger than one round of the grid: every block takes many
    tiles, segments and chunks of each pass in turn (147 tensors, 86.6 M
    parameters)."""
    w = W.get_workload("vit_b16")
    say(f"[single] vit_b16 impl {impl}")
    a = run(w, impl, SINGLE, 2)
    b = run(w, impl, SPLIT, 2)
    assert_same(a, b, f"vit_b16 impl {impl}")


def test_ragged_many_small_tensors_bitwise():
    """2,000 small tensors (more finalize items than the grid has blocks)."""
    rng = np.random.default_rng(163)
    shapes = []
    for _ in range(2000):
        n = int(round(np.exp(rng.uniform(np.log(16), np.log(4000)))))
        if rng.random() < 0.5:
            shapes.append((n,))
        else:
            r = max(1, int(round(np.sqrt(n * np.exp(rng.uniform(-2, 2))))))
            shapes.append((r, max(1, n // r)))
    w = W.custom_workload("single_ragged", shapes, grad_std=1e-3, steps=2, wid=164)
    a = run(w, L.LOPT_MLP_AUTO, SINGLE, 2)
    b = run(w, L.LOPT_MLP_AUTO, SPLIT, 2)
    assert_same(a, b, "ragged 2000")


def test_one_launch_against_the_oracle():
    """Parity with the oracle on the one-launch step directly (edge shapes,
    five steps, default path)."""
    w = W.custom_workload("single_oracle", MIXED, grad_std=1e-2, steps=5, wid=165)
    cfg = L.config_from(launch=SINGLE)
    weights = W.mlp_weights(11, bias_std=0.1)
    pa, sa, _, t, mode = run(w, L.LOPT_MLP_AUTO, SINGLE, 5)
    assert mode == SINGLE and t == 5
    want = oracle_run(w, weights, hyper_from_cfg(cfg), 5)
    errs = []
    for i, tt in enumerate(w.tensors):
        st = sa[i].cpu().numpy()
        n, R, C = tt.rows * tt.cols, tt.rows, tt.cols
        got = {"p": pa[i].cpu().numpy().reshape(R, C), "m": st[:3 * n].reshape(3, R, C), "v": st[3 * n:4 * n].reshape(R, C),
               "r": st[4 * n:4 * n + 3 * R].reshape(3, R), "c": st[4 * n + 3 * R:].reshape(3, C)}
        errs += compare(got, want[i], f"single_oracle[{i}]")
    assert not errs, "\n".join(errs[:20])


@pytest.mark.parametrize("launch", [SINGLE, SPLIT])
def test_graph_replay_equals_eager(launch):
    shapes = [(64, 96), (1, 500), (300, 7)]
    m = W.mlp_weights(11, bias_std=0.1)
    w = W.custom_workload("single_graph", shapes, steps=5, wid=166)
    grads = [torch.from_numpy(W.grad_at(w, i, 1).reshape(t.shape)).cuda() for i, t in enumerate(w.tensors)]

    def fresh():
        ps = [torch.from_numpy(W.param_init(w, i).reshape(t.shape)).cuda() for i, t in enumerate(w.tensors)]
        return ps, L.LOpt(ps, m, L.config_from(launch=launch))

    pe, eager = fresh()
    pg, graphed = fresh()
    eager.step(grads)
    graphed.step(grads)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        graphed.step(grads)
    for k in range(2, 7):
        eager.step(grads)
        g.replay()
        torch.cuda.synchronize()
        for i in range(len(shapes)):
            assert torch.equal(pe[i], pg[i]), (k, i)
            assert torch.equal(eager.states[i], graphed.states[i]), (k, i)
    assert eager.t == 6 and graphed.t == 6
    eager.close()
    graphed.close()


def test_timing_events_of_a_one_launch_step():
    p = torch.zeros(64, 64, device="cuda")
    opt = L.LOpt([p], W.mlp_weights(), L.config_from(launch=SINGLE))
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(L.LOPT_N_KERNELS + 1)]
    for e in ev:          # torch creates the HIP event on its first record
        e.record()
    L.lopt_set_timing_events(opt.handle, [e.cuda_event for e in ev])
    opt.step([torch.full((64, 64), 1e-3, device="cuda")])
    L.lopt_set_timing_events(opt.handle, [])
    torch.cuda.synchronize()
    whole = ev[L.LOPT_N_KERNELS - 1].elapsed_time(ev[L.LOPT_N_KERNELS])
    assert whole > 0 and ev[0].elapsed_time(ev[L.LOPT_N_KERNELS]) >= whole
    assert opt.t == 1
    opt.close()
