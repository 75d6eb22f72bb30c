"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bar: |gpu - oracle| <= 1e-7 + 1e-5 |oracle| element-wise on p, m1..m3, v,
r1..r3 and c1..c3 after each case's step count.  Integer/bitwise properties
(determinism, resume, tensor independence) are checked bit for bit.
"""
import numpy as np
import pytest

import oracle
from gpu_harness import IMPLS, DeviceRun, compare, hyper_from_cfg, oracle_run, parity, parity_one_step_rows, say

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("no GPU", allow_module_level=True)

from learned_optimizer_step_amd import lopt as L  # noqa: E402
from learned_optimizer_step_amd import workloads as W  # noqa: E402


EDGE_SHAPES = [(1,), (2,), (3,), (15,), (16,), (17,), (63,), (65,), (40000,),
               (1, 1), (2, 3), (3, 1), (7, 1), (17, 33), (65, 3), (4, 513), (300, 2),
               (129, 257), (600, 5), (5, 600), (1000, 1), (33, 64)]


# 2-D shapes whose column count is a multiple of 64: every 64-element wave
# iteration of the matrix-core apply kernel lies inside one row, and the row
# features enter through the row-term slot
ROW_UNIFORM_SHAPES = [(2, 64), (3, 128), (5, 192), (64, 64), (100, 320), (7, 4096), (300, 256)]

# 2-D shapes whose column count is above 64 and not a multiple of it: the row
# features enter as three slots, some wave iterations lie inside one row and
# the others span two rows
MIXED_ROW_SHAPES = [(9, 65), (40, 100), (17, 127), (12, 200), (6, 1000), (3, 4097), (70, 96), (2, 1025)]


def mlp(n_time=11, bias_std=0.0):
    return W.mlp_weights(n_time, bias_std=bias_std)


def check(errs):
    assert not errs, "\n".join(errs[:20])


@pytest.mark.parametrize("impl", IMPLS)
def test_single256_ten_steps(impl):
    w = W.get_workload("single256")
    check(parity(w, mlp(), L.config_from(mlp_impl=impl), torch))


@pytest.mark.parametrize("impl", IMPLS)
def test_edge_shapes_ten_steps(impl):
    w = W.custom_workload("edges", EDGE_SHAPES, grad_std=1e-2, steps=10, wid=101)
    check(parity(w, mlp(bias_std=0.1), L.config_from(mlp_impl=impl), torch))


MATRIX_IMPLS = [L.LOPT_MLP_BF16X8, L.LOPT_MLP_BF16X9, L.LOPT_MLP_MFMA, L.LOPT_MLP_BF16X6, L.LOPT_MLP_FP16X3]


@pytest.mark.parametrize("impl", MATRIX_IMPLS)
@pytest.mark.parametrize("n_feat", [L.LOPT_N_FEATURES, L.LOPT_VELO_FEATURES])
def test_row_uniform_shapes_ten_steps(n_feat, impl):
    w = W.custom_workload("rowuni", ROW_UNIFORM_SHAPES, grad_std=1e-2, steps=10, wid=104)
    weights = W.mlp_weights(11, bias_std=0.1, n_feat=n_feat)
    check(parity(w, weights, L.config_from(mlp_impl=impl, n_feat=n_feat), torch))


@pytest.mark.parametrize("impl", MATRIX_IMPLS)
@pytest.mark.parametrize("n_feat", [L.LOPT_N_FEATURES, L.LOPT_VELO_FEATURES])
def test_mixed_row_shapes_ten_steps(n_feat, impl):
    w = W.custom_workload("mixrow", MIXED_ROW_SHAPES, grad_std=1e-2, steps=10, wid=150)
    weights = W.mlp_weights(11, bias_std=0.1, n_feat=n_feat)
    check(parity(w, weights, L.config_from(mlp_impl=impl, n_feat=n_feat), torch))


# paths whose products are exact and accumulated in fp32, and the narrower ones
FP32_IMPLS = (L.LOPT_MLP_BF16X8, L.LOPT_MLP_BF16X9, L.LOPT_MLP_MFMA, L.LOPT_MLP_VALU)
NARROW_IMPLS = (L.LOPT_MLP_BF16X6, L.LOPT_MLP_FP16X3)


def test_update_accuracy_of_each_mlp_path():
    """The MLP's accuracy, seen through the update: with p = 0 (so no decay
    term), one step leaves p = -lr step_mult dir exp(exp_mult mag), the MLP
    output rounded once to fp32.  Over the elements whose update is not tiny
    (>= 1e-3 of the largest; smaller ones come from cancellation in the last
    layer), on three seeded weight draws:
      * against the fp64 oracle, the bf16 paths with fp32 arithmetic (bf16x9:
        exact products from bf16 pieces; bf16x8: each product within 2^-30 of
        itself; fp32 accumulation) are at the fp32 paths' level: rms error
        within 1.15x and max error within 1.5x of the larger of the two fp32
        paths' (the matrix-core and the vector-ALU path, which compute the same
        fp32 products in different summation orders);
      * the narrower paths (bf16x6, fp16x3) stay within 1.5x (rms) and 4x
        (max) of the fp32 paths;
      * against the fp32 matrix path on identical inputs (evaluation only),
        bf16x8 and bf16x9 differ no more than the vector-ALU path does (1.25x,
        rms)."""
    shapes = [(256, 256), (4096,), (100, 300), (64, 128), (33, 65)]
    w = W.custom_workload("updacc", shapes, param_std=0.0, grad_std=1e-2, steps=1, wid=176)
    for seed in ((0, 9999), (5, 1), (5, 2)):
        weights = W.mlp_weights(11, seed=seed, bias_std=0.1)
        want = oracle_run(w, weights, hyper_from_cfg(L.config_from()), 1)
        ref = np.concatenate([np.asarray(want[i]["p"], np.float64).ravel() for i in range(len(shapes))])
        keep = np.zeros(ref.size, bool)
        off = 0
        for i in range(len(shapes)):
            r = np.asarray(want[i]["p"], np.float64).ravel()
            keep[off:off + r.size] = np.abs(r) >= 1e-3 * np.abs(r).max()
            off += r.size
        got = {}
        for impl in IMPLS:
            run = DeviceRun(w, weights, L.config_from(mlp_impl=impl), torch)
            run.step(1)
            got[impl] = np.concatenate([np.asarray(run.fetch(i)["p"], np.float64).ravel()
                                        for i in range(len(shapes))])
            run.close()

        def rel(a, b):
            e = np.abs(a[keep] - b[keep]) / np.abs(b[keep])
            return float(np.sqrt(np.mean(e ** 2))), float(e.max())

        vs_oracle = {impl: rel(got[impl], ref) for impl in IMPLS}
        vs_mfma = {impl: rel(got[impl], got[L.LOPT_MLP_MFMA]) for impl in IMPLS if impl != L.LOPT_MLP_MFMA}
        for impl in IMPLS:
            say(f"[update accuracy] weights {seed} impl {impl} vs oracle: rms {vs_oracle[impl][0]:.3e}, "
                f"max {vs_oracle[impl][1]:.3e}" + (f"; vs fp32 matrix path: rms {vs_mfma[impl][0]:.3e}, "
                                                  f"max {vs_mfma[impl][1]:.3e}" if impl in vs_mfma else "")
                + f" ({int(keep.sum())} elements)")
        rms32 = max(vs_oracle[L.LOPT_MLP_MFMA][0], vs_oracle[L.LOPT_MLP_VALU][0])
        max32 = max(vs_oracle[L.LOPT_MLP_MFMA][1], vs_oracle[L.LOPT_MLP_VALU][1])
        for impl in (L.LOPT_MLP_BF16X8, L.LOPT_MLP_BF16X9):
            assert vs_oracle[impl][0] <= 1.15 * rms32 and vs_oracle[impl][1] <= 1.5 * max32, (seed, impl, vs_oracle)
            assert vs_mfma[impl][0] <= 1.25 * vs_mfma[L.LOPT_MLP_VALU][0], (seed, impl, vs_mfma)
        for impl in NARROW_IMPLS:
            assert vs_oracle[impl][0] <= 1.5 * rms32 and vs_oracle[impl][1] <= 4.0 * max32, (seed, vs_oracle)


def test_auto_runs_bf16x8():
    """LOPT_MLP_AUTO resolves to the bf16x8 path for any weights (its result
    identical to an explicit LOPT_MLP_BF16X8), including weights the fp16x3
    path refuses (a W1 entry of 40000)."""
    w = W.custom_workload("auto", [(64, 128), (300,)], param_std=0.02, grad_std=1e-2, steps=2, wid=180)
    weights = W.mlp_weights(11, bias_std=0.1)
    big = weights.copy()
    big[5] = 40000.0
    for mlp in (weights, big):
        out = {}
        for impl in (L.LOPT_MLP_AUTO, L.LOPT_MLP_BF16X8):
            run = DeviceRun(w, mlp, L.config_from(mlp_impl=impl), torch)
            assert L.lopt_get_mlp_impl(run.opt.handle) == L.LOPT_MLP_BF16X8
            for t in (1, 2):
                run.step(t)
            out[impl] = [run.fetch(i)["p"] for i in range(len(w.tensors))]
            run.close()
        for a, b in zip(out[L.LOPT_MLP_AUTO], out[L.LOPT_MLP_BF16X8]):
            assert np.array_equal(np.asarray(a), np.asarray(b))


@pytest.mark.parametrize("impl", IMPLS)
@pytest.mark.parametrize("scale", ["large", "small"])
def test_magnitudes_far_from_one(impl, scale):
    """Parameters many orders of magnitude from 1 (1e6 or 1e-8) and gradients
    of 1e-2 or 1e-12: one element's features then span a wide range of
    exponents, which the bf16x6 path's pieces must follow exactly.  (The
    gradients stay small: an EMA of 1e3-sized gradients that cancels towards
    zero carries an fp32 error of ~1e-5 absolute, above the parity bar's
    absolute term, on every path and whatever the MLP does.)"""
    p_std, g_std = (1e6, 1e-2) if scale == "large" else (1e-8, 1e-12)
    w = W.custom_workload(f"mag_{scale}", [(64, 64), (300,), (40, 100), (3, 257)], param_std=p_std,
                          grad_std=g_std, steps=5, wid=177)
    check(parity(w, mlp(bias_std=0.1), L.config_from(mlp_impl=impl), torch))


@pytest.mark.parametrize("impl", IMPLS)
def test_mlp_weights_four_times_larger(impl):
    """The test MLP's weights and biases scaled by 4: hidden activations and
    every operand the matrix paths split move further from 1 (and layer 3's
    output into the range where exp(mag exp_mult) matters more)."""
    w = W.custom_workload("bigw", [(64, 128), (3000,), (33, 65), (200, 7)], grad_std=1e-2, steps=5, wid=178)
    weights = (4.0 * mlp(bias_std=0.2)).astype(np.float32)
    check(parity(w, weights, L.config_from(mlp_impl=impl), torch))


@pytest.mark.parametrize("impl", IMPLS)
def test_first_layer_outputs_beyond_fp16_range(impl):
    """First-layer weights of the per-element features (all but the row and
    step features) 20000 times the test MLP's: about 1 % of the hidden
    activations exceed 2^15 and the largest exceed fp16's largest value
    (checked on the oracle's own activations), so the fp16x3 path must rescale
    those waves.  lr and exp_mult are divided by 20000 too, which keeps the
    update near the unscaled MLP's and its conditioning the usual one."""
    S = 20000.0
    w = W.custom_workload("bigh1", [(64, 256), (2048,), (40, 100)], grad_std=1e-2, steps=2, wid=179)
    weights = mlp(bias_std=0.1).copy()
    w1 = weights[:32 * (L.LOPT_N_FEATURES + 11)].reshape(32, -1)
    w1[:, [f for f in range(L.LOPT_N_FEATURES) if f not in (13, 14, 15)]] *= S
    d = L.lopt_default_config()
    cfg = L.config_from(mlp_impl=impl, lr=1.0 / S, exp_mult=d.exp_mult / S)
    hp = hyper_from_cfg(cfg).as_f32()
    m = oracle.unpack_mlp(weights, hp.n_time, hp.n_feat)
    _, _, info = oracle.step_tensor(W.param_init(w, 0), W.grad_at(w, 0, 1), W.state_init(w, 0), 1, m, hp, keep=True)
    h1 = np.maximum(info.x.reshape(-1, info.x.shape[-1]) @ m.W1.T + m.b1, 0.0)
    assert h1.max() > 65504.0, h1.max()
    check(parity(w, weights, cfg, torch))


@pytest.mark.parametrize("impl", IMPLS)
def test_no_time_features_lr_wd_prewarmed(impl):
    w = W.custom_workload("nt0", [(37, 41), (1, 77), (9,)], grad_std=1e-3, steps=4,
                          prewarm_std=1e-3, wid=102)
    cfg = L.config_from(mlp_impl=impl, n_time=0, lr=0.5, weight_decay=0.01, exp_mult=0.05, step_mult=0.01)
    check(parity(w, mlp(n_time=0, bias_std=0.2), cfg, torch))


@pytest.mark.parametrize("impl", IMPLS)
def test_zero_gradients_stay_finite(impl):
    w = W.custom_workload("zeros", [(8, 8), (1, 5)], grad_std=0.0, steps=3, wid=103)
    check(parity(w, mlp(bias_std=0.1), L.config_from(mlp_impl=impl), torch))


def sample_rows(R, k, seed):
    rng = np.random.default_rng(seed)
    return sorted(set([0, R - 1] + rng.choice(R, min(R, k), replace=False).tolist()))


def _run_states(w, cfg, steps, m):
    run = DeviceRun(w, m, cfg, torch)
    for t in range(1, steps + 1):
        run.step(t)
    out = [run.fetch(i) for i in range(len(w.tensors))]
    run.close()
    return out


def test_bitwise_deterministic():
    w = W.custom_workload("det", [(300, 200), (1, 5000), (1000, 3)], steps=3, wid=104)
    m = mlp(bias_std=0.1)
    a = _run_states(w, L.config_from(), 3, m)
    b = _run_states(w, L.config_from(), 3, m)
    for x, y in zip(a, b):
        for k in x:
            assert np.array_equal(x[k], y[k]), k


def test_list_equals_separate_calls():
    shapes = [(70, 90), (1, 333), (5, 1)]
    m = mlp(bias_std=0.1)
    w = W.custom_workload("ind", shapes, steps=2, wid=105)
    together = _run_states(w, L.config_from(), 2, m)
    for i, tt in enumerate(w.tensors):
        p = torch.from_numpy(W.param_init(w, i).reshape(tt.shape)).cuda()
        opt = L.LOpt([p], m, L.config_from())
        for t in (1, 2):
            opt.step([torch.from_numpy(W.grad_at(w, i, t).reshape(tt.shape)).cuda()])
        torch.cuda.synchronize()
        v = opt.state_views(0)
        assert np.array_equal(p.cpu().numpy().reshape(tt.rows, tt.cols), together[i]["p"]), i
        for k in ("m", "v", "r", "c"):
            assert np.array_equal(v[k].cpu().numpy(), together[i][k]), (i, k)
        opt.close()


def test_resume_equals_uninterrupted_and_grad_pointers_may_change():
    shapes = [(40, 50), (1, 64)]
    m = mlp(bias_std=0.1)
    w = W.custom_workload("res", shapes, steps=10, wid=106)
    full = _run_states(w, L.config_from(), 10, m)
    run = DeviceRun(w, m, L.config_from(), torch)
    for t in range(1, 6):
        run.step(t)          # fresh gradient tensors each step: pointers change
    saved = [run.fetch(i) for i in range(len(shapes))]
    run.close()
    run2 = DeviceRun(w, m, L.config_from(), torch)
    for i in range(len(shapes)):
        run2.params[i].copy_(torch.from_numpy(saved[i]["p"].reshape(w.tensors[i].shape)))
        v = run2.opt.state_views(i)
        for k in ("m", "v", "r", "c"):
            v[k].copy_(torch.from_numpy(saved[i][k]))
    run2.opt.t = 5
    for t in range(6, 11):
        run2.step(t)
    assert run2.opt.t == 10
    for i in range(len(shapes)):
        got = run2.fetch(i)
        for k in got:
            assert np.array_equal(got[k], full[i][k]), (i, k)
    run2.close()


def test_grad_pointer_changes_queued_without_waiting():
    # gradients of steps 1..8 staged on the device first, then eight steps
    # queued back to back, each with a different gradient tensor: every step
    # must read its own pointers (the pinned slots are reused from step 3 on)
    shapes = [(48, 80), (1, 300), (7, 129)]
    m = mlp(bias_std=0.1)
    w = W.custom_workload("gptr", shapes, grad_std=1e-2, steps=8, wid=160)
    # reference: one gradient buffer per tensor for all steps (pointers never change)
    ref_params = [torch.from_numpy(W.param_init(w, i).reshape(t.shape)).cuda() for i, t in enumerate(w.tensors)]
    fixed = [torch.empty(t.shape, device="cuda") for t in w.tensors]
    ref_opt = L.LOpt(ref_params, m, L.config_from())
    for t in range(1, 9):
        for i, tt in enumerate(w.tensors):
            fixed[i].copy_(torch.from_numpy(W.grad_at(w, i, t).reshape(tt.shape)))
        ref_opt.step(fixed)
    torch.cuda.synchronize()
    ref = []
    for i, tt in enumerate(w.tensors):
        v = ref_opt.state_views(i)
        ref.append({k: v[k].cpu().numpy() for k in ("m", "v", "r", "c")})
        ref[-1]["p"] = ref_params[i].cpu().numpy().reshape(tt.rows, tt.cols)
    ref_opt.close()
    params = [torch.from_numpy(W.param_init(w, i).reshape(t.shape)).cuda() for i, t in enumerate(w.tensors)]
    staged = [[torch.from_numpy(W.grad_at(w, i, t).reshape(tt.shape)).cuda() for i, tt in enumerate(w.tensors)]
              for t in range(1, 9)]
    opt = L.LOpt(params, m, L.config_from())
    torch.cuda.synchronize()
    for t in range(8):
        opt.step(staged[t])
    torch.cuda.synchronize()
    assert opt.t == 8
    for i, tt in enumerate(w.tensors):
        v = opt.state_views(i)
        assert np.array_equal(params[i].cpu().numpy().reshape(tt.rows, tt.cols), ref[i]["p"]), i
        for k in ("m", "v", "r", "c"):
            assert np.array_equal(v[k].cpu().numpy(), ref[i][k]), (i, k)
    opt.close()


def test_step_rejects_a_different_list():
    p = torch.zeros(4, 4, device="cuda")
    q = torch.zeros(4, 4, device="cuda")
    opt = L.LOpt([p], mlp(), L.config_from())
    g = torch.zeros(4, 4, device="cuda")
    with pytest.raises(L.LoptError) as e:
        L.lopt_step(opt.handle, [L.lopt_tensor(q.data_ptr(), g.data_ptr(), opt.states[0].data_ptr(), 4, 4)],
                    torch.cuda.current_stream().cuda_stream)
    assert e.value.status == L.LOPT_ERR_STATE
    assert opt.t == 0
    opt.close()


def test_lr_schedule_and_weight_decay_through_torch_optimizer():
    shapes = [(48, 40), (1, 100)]
    m = mlp(bias_std=0.1)
    w = W.custom_workload("sched", shapes, steps=6, wid=107)
    params = [torch.from_numpy(W.param_init(w, i).reshape(t.shape)).cuda() for i, t in enumerate(w.tensors)]
    opt = L.LearnedOptimizer(params, m, lr=0.8, weight_decay=0.05)
    sched = torch.optim.lr_scheduler.CosineAnnealingLR(opt, T_max=6)
    ps = [W.param_init(w, i) for i in range(2)]
    sts = [W.state_init(w, i) for i in range(2)]
    for t in range(1, 7):
        lr = opt.param_groups[0]["lr"]
        gs = [W.grad_at(w, i, t) for i in range(2)]
        for p, g, tt in zip(params, gs, w.tensors):
            p.grad = torch.from_numpy(g.reshape(tt.shape)).cuda()
        opt.step()
        ps, sts = oracle.step(ps, gs, sts, t, m, oracle.Hyper(lr=lr, weight_decay=0.05))
        sched.step()
    torch.cuda.synchronize()
    assert opt.lopt.t == 6
    errs = []
    for i, tt in enumerate(w.tensors):
        v = opt.lopt.state_views(i)
        got = {"p": params[i].cpu().numpy().reshape(tt.rows, tt.cols)}
        got.update({k: v[k].cpu().numpy() for k in ("m", "v", "r", "c")})
        errs += compare(got, dict(p=ps[i], **sts[i]), f"sched[{i}]")
    check(errs)


@pytest.mark.parametrize("impl", IMPLS)
def test_per_tensor_lr_and_weight_decay(impl):
    # every tensor its own (lr, wd), through lopt_set_tensor_hyper, 5 steps
    shapes = [(40, 64), (1, 300), (33, 17), (7,), (5, 129)]
    w = W.custom_workload("th", shapes, grad_std=1e-2, steps=5, wid=170)
    th = [(0.8, 0.05), (1.5, 0.0), (0.3, 0.2), (1.0, 0.01), (2.0, 0.1)]
    check(parity(w, mlp(bias_std=0.1), L.config_from(mlp_impl=impl, lr=0.5, weight_decay=0.3), torch,
                 tensor_hyper=th))


def test_per_tensor_values_equal_to_the_config_are_bitwise_the_config():
    # per-tensor pairs built from the same fp32 expressions as the list-wide ones;
    # clearing them goes back to the config's values
    shapes = [(48, 64), (1, 200), (9, 31)]
    w = W.custom_workload("th_eq", shapes, grad_std=1e-2, steps=3, wid=171)
    m = mlp(bias_std=0.1)
    cfg = L.config_from(lr=0.7, weight_decay=0.05)
    a = DeviceRun(w, m, cfg, torch)
    b = DeviceRun(w, m, cfg, torch)
    b.opt.set_tensor_hyper([0.7] * 3, [0.05] * 3)
    for t in (1, 2):
        a.step(t)
        b.step(t)
    b.opt.set_tensor_hyper(None, None)
    a.step(3)
    b.step(3)
    for i in range(len(shapes)):
        x, y = a.fetch(i), b.fetch(i)
        for k in x:
            assert np.array_equal(x[k], y[k]), (i, k)
    with pytest.raises(ValueError):
        b.opt.set_tensor_hyper([0.1, 0.2], [0.0, 0.0])          # the binding checks the count
    with pytest.raises(ValueError):
        b.opt.set_tensor_hyper([0.1] * 3, None)
    with pytest.raises(L.LoptError) as e:                       # so does the library
        L.lopt_set_tensor_hyper(b.opt.handle, [0.1, 0.2], [0.0, 0.0])
    assert e.value.status == L.LOPT_ERR_STATE
    with pytest.raises(L.LoptError) as e:
        b.opt.set_tensor_hyper([float("nan")] * 3, [0.0] * 3)
    assert e.value.status == L.LOPT_ERR_INVALID_ARGUMENT
    a.close()
    b.close()


def test_parameter_groups_with_a_schedule_through_torch_optimizer():
    # two groups, as a training script makes them: weights with weight decay,
    # biases and norms without; a cosine schedule changes both groups' lr every
    # step, so the per-tensor values are sent at every step
    shapes = [(48, 40), (40,), (1, 100), (64, 32)]
    m = mlp(bias_std=0.1)
    w = W.custom_workload("groups", shapes, steps=6, wid=172)
    params = [torch.from_numpy(W.param_init(w, i).reshape(t.shape)).cuda() for i, t in enumerate(w.tensors)]
    decay, no_decay = [params[0], params[3]], [params[1], params[2]]
    opt = L.LearnedOptimizer([{"params": decay, "weight_decay": 0.05}, {"params": no_decay, "weight_decay": 0.0}],
                             m, lr=0.8)
    sched = torch.optim.lr_scheduler.CosineAnnealingLR(opt, T_max=6)
    order = decay + no_decay           # the library's tensor order: group by group
    idx = [next(i for i, p in enumerate(params) if p is q) for q in order]
    ps = [W.param_init(w, i) for i in idx]
    sts = [W.state_init(w, i) for i in idx]
    for t in range(1, 7):
        th = [(g["lr"], g["weight_decay"]) for g in opt.param_groups for _ in g["params"]]
        gs = [W.grad_at(w, i, t) for i in idx]
        for q, g, i in zip(order, gs, idx):
            q.grad = torch.from_numpy(g.reshape(w.tensors[i].shape)).cuda()
        opt.step()
        ps, sts = oracle.step(ps, gs, sts, t, m, oracle.Hyper(), tensor_hyper=th)
        sched.step()
    torch.cuda.synchronize()
    errs = []
    for j, i in enumerate(idx):
        tt = w.tensors[i]
        v = opt.lopt.state_views(j)
        got = {"p": params[i].cpu().numpy().reshape(tt.rows, tt.cols)}
        got.update({k: v[k].cpu().numpy() for k in ("m", "v", "r", "c")})
        errs += compare(got, dict(p=ps[j], **sts[j]), f"groups[{i}]")
    check(errs)


def test_nd_and_scalar_parameters_through_torch_optimizer():
    # a convolution weight, a scalar, a vector and a matrix, as a model's
    # parameters() gives them; the library sees each as its matrix view
    nd = [(8, 3, 5, 5), (), (7,), (6, 10)]
    mats = [L.matrix_shape(x) for x in nd]
    w = W.custom_workload("nd", [m if m[0] > 1 else (m[1],) for m in mats], grad_std=1e-2, steps=4, wid=173)
    m = mlp(bias_std=0.1)
    params = [torch.from_numpy(W.param_init(w, i).reshape(x)).cuda() for i, x in enumerate(nd)]
    opt = L.LearnedOptimizer(params, m, lr=0.9, weight_decay=0.02)
    ps = [W.param_init(w, i) for i in range(len(nd))]
    sts = [W.state_init(w, i) for i in range(len(nd))]
    for t in range(1, 5):
        gs = [W.grad_at(w, i, t) for i in range(len(nd))]
        for p, g, x in zip(params, gs, nd):
            p.grad = torch.from_numpy(g.reshape(x)).cuda()
        opt.step()
        ps, sts = oracle.step(ps, gs, sts, t, m, oracle.Hyper(lr=0.9, weight_decay=0.02))
    torch.cuda.synchronize()
    errs = []
    for i, (r, c) in enumerate(mats):
        v = opt.lopt.state_views(i)
        got = {"p": params[i].cpu().numpy().reshape(r, c)}
        got.update({k: v[k].cpu().numpy() for k in ("m", "v", "r", "c")})
        errs += compare(got, dict(p=ps[i], **sts[i]), f"nd[{i}:{nd[i]}]")
    check(errs)


@pytest.mark.parametrize("impl", IMPLS)
def test_tensors_without_gradient_are_skipped(impl):
    # some tensors have no gradient in some steps (None, as torch gives a
    # parameter that took no part in the loss): they stay as they are, the
    # others step as usual; step 4 has no gradient at all
    shapes = [(40, 64), (1, 300), (33, 17), (7,)]
    w = W.custom_workload("skip", shapes, grad_std=1e-2, steps=5, wid=174)
    m = mlp(bias_std=0.1)
    missing = {1: {1}, 2: {0, 3}, 3: {2}, 4: {0, 1, 2, 3}, 5: set()}
    params = [torch.from_numpy(W.param_init(w, i).reshape(t.shape)).cuda() for i, t in enumerate(w.tensors)]
    opt = L.LOpt(params, m, L.config_from(mlp_impl=impl))
    ps = [W.param_init(w, i) for i in range(len(shapes))]
    sts = [W.state_init(w, i) for i in range(len(shapes))]
    for t in range(1, 6):
        gs = [None if i in missing[t] else W.grad_at(w, i, t) for i in range(len(shapes))]
        opt.step([None if g is None else torch.from_numpy(g.reshape(tt.shape)).cuda()
                  for g, tt in zip(gs, w.tensors)])
        ps, sts = oracle.step(ps, gs, sts, t, m, hyper_from_cfg(opt.cfg))
    torch.cuda.synchronize()
    assert opt.t == 5
    errs = []
    for i, tt in enumerate(w.tensors):
        v = opt.state_views(i)
        got = {"p": params[i].cpu().numpy().reshape(tt.rows, tt.cols)}
        got.update({k: v[k].cpu().numpy() for k in ("m", "v", "r", "c")})
        errs += compare(got, dict(p=ps[i], **sts[i]), f"skip[{i}]")
    check(errs)
    opt.close()


def test_graph_replay_matches_eager_steps():
    shapes = [(64, 96), (1, 500), (300, 7)]
    m = mlp(bias_std=0.1)
    w = W.custom_workload("graph", shapes, steps=5, wid=108)
    grads = [torch.from_numpy(W.grad_at(w, i, 1).reshape(t.shape)).cuda() for i, t in enumerate(w.tensors)]

    def fresh():
        ps = [torch.from_numpy(W.param_init(w, i).reshape(t.shape)).cuda() for i, t in enumerate(w.tensors)]
        return ps, L.LOpt(ps, m, L.config_from())

    pe, eager = fresh()
    pg, graphed = fresh()
    eager.step(grads)
    graphed.step(grads)          # binds the gradient pointers outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        graphed.step(grads)
    for k in range(2, 6):
        eager.step(grads)
        g.replay()
        torch.cuda.synchronize()
        for i in range(len(shapes)):
            assert torch.equal(pe[i], pg[i]), (k, i)
            assert torch.equal(eager.states[i], graphed.states[i]), (k, i)
    assert eager.t == 5 and graphed.t == 5
    eager.close()
    graphed.close()


def test_set_config_rejects_other_n_time_and_timing_events_api():
    p = torch.zeros(8, 8, device="cuda")
    opt = L.LOpt([p], mlp(), L.config_from())
    with pytest.raises(L.LoptError):
        L.lopt_set_config(opt.handle, L.config_from(n_time=0))
    L.lopt_set_config(opt.handle, L.config_from(lr=0.5))
    with pytest.raises(L.LoptError):
        L.lopt_set_timing_events(opt.handle, [1, 2])
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(L.LOPT_N_KERNELS + 1)]
    for e in ev:
        e.record()
    L.lopt_set_timing_events(opt.handle, [e.cuda_event for e in ev])
    opt.step([torch.full((8, 8), 1e-3, device="cuda")])
    L.lopt_set_timing_events(opt.handle, [])
    torch.cuda.synchronize()
    times = [ev[j].elapsed_time(ev[j + 1]) for j in range(L.LOPT_N_KERNELS)]
    assert all(t >= 0 for t in times)
    opt.close()


def test_empty_tensor_list_steps():
    opt = L.LOpt([], mlp(), L.config_from())
    opt.step([])
    assert opt.t == 0     # no kernels, so the device counter does not advance
    opt.close()


# ----------------------------------------------------------------- VeLO-shaped variant
VNF = L.LOPT_VELO_FEATURES


def vmlp(n_time=11, bias_std=0.1):
    return W.mlp_weights(n_time, bias_std=bias_std, n_feat=VNF)


@pytest.mark.parametrize("impl", IMPLS)
def test_velo_shaped_edges_and_256_ten_steps(impl):
    w = W.custom_workload("velo_edges", EDGE_SHAPES + [(256, 256)], grad_std=1e-2, steps=10, wid=110)
    check(parity(w, vmlp(), L.config_from(mlp_impl=impl, n_feat=VNF), torch))


@pytest.mark.parametrize("impl", IMPLS)
def test_velo_shaped_vit_b16_subset_prewarmed_lr_wd(impl):
    w = W.get_workload("vit_b16")
    names = [t.name for t in w.tensors]
    subset = [names.index(n) for n in ("pos_embed", "blocks.3.qkv.weight", "blocks.3.qkv.bias", "head")]
    cfg = L.config_from(mlp_impl=impl, n_feat=VNF, lr=0.8, weight_decay=0.02)
    check(parity(w, vmlp(), cfg, torch, steps=3, subset=subset))


def test_velo_shaped_one_step_sampled_llama_rows():
    w = W.get_workload("llama1b")
    names = [t.name for t in w.tensors]
    picks = {names.index("layers.7.gate"): sample_rows(2048, 16, 11), names.index("layers.7.mlp_norm"): None}
    check(parity_one_step_rows(w, vmlp(), L.config_from(n_feat=VNF), torch, picks))


def test_set_config_keeps_the_feature_count():
    p = torch.zeros(4, 4, device="cuda")
    opt = L.LOpt([p], vmlp(), L.config_from(n_feat=VNF))
    with pytest.raises(L.LoptError):
        L.lopt_set_config(opt.handle, L.config_from(n_feat=L.LOPT_N_FEATURES))
    with pytest.raises(ValueError):       # weights sized for the other variant
        L.LOpt([p], mlp(), L.config_from(n_feat=VNF))
    opt.close()


@pytest.mark.parametrize("impl", IMPLS)
@pytest.mark.parametrize("bad", [float("nan"), float("inf")])
def test_non_finite_gradient_stays_in_its_tensor(impl, bad):
    # Reading R23: non-finite inputs are not checked.  One bad gradient element
    # of tensor 0 must show up in exactly the accumulators the step definition
    # routes it to (its m and v, its row's r, its column's c), equal to the
    # oracle everywhere else; tensor 1 of the same step is untouched by it.
    # The parameters of tensor 0 are not compared (its per-tensor statistics
    # are non-finite; the ReLU of a NaN is unspecified on the GPU).
    shapes = [(12, 40), (9, 33)]
    w = W.custom_workload("nonfinite", shapes, grad_std=1e-2, steps=1, wid=130)
    cfg = L.config_from(mlp_impl=impl)
    weights = mlp(bias_std=0.1)
    run = DeviceRun(w, weights, cfg, torch)
    grads = [torch.from_numpy(W.grad_at(w, i, 1).reshape(t.shape)).cuda() for i, t in enumerate(w.tensors)]
    grads[0][5, 17] = bad
    run.opt.step(grads)
    got = [run.fetch(i) for i in range(2)]
    run.close()
    hp = hyper_from_cfg(cfg)
    g0 = W.grad_at(w, 0, 1).reshape(shapes[0]).copy()
    g0[5, 17] = bad
    gs = [g0, W.grad_at(w, 1, 1).reshape(shapes[1])]
    with np.errstate(all="ignore"):    # the oracle's arithmetic on the bad element
        ps, sts = oracle.step([W.param_init(w, i) for i in range(2)], gs,
                              [W.state_init(w, i) for i in range(2)], 1, weights, hp)
    check(compare(got[1], dict(p=ps[1], **sts[1]), "clean tensor"))
    want = sts[0]
    errs = []
    for k in ("m", "v", "r", "c"):
        a, b = np.asarray(got[0][k], np.float64), np.asarray(want[k], np.float64).reshape(got[0][k].shape)
        if not (np.array_equal(np.isnan(a), np.isnan(b)) and np.array_equal(np.isposinf(a), np.isposinf(b))
                and np.array_equal(np.isneginf(a), np.isneginf(b))):
            errs.append(f"{k}: non-finite pattern differs ({int((~np.isfinite(a)).sum())} vs {int((~np.isfinite(b)).sum())})")
            continue
        fin = np.isfinite(b)
        assert (~fin).any()
        bound = 1e-7 + 1e-5 * np.abs(b[fin])
        if not np.all(np.abs(a[fin] - b[fin]) <= bound):
            errs.append(f"{k}: finite entries out of tolerance")
    check(errs)


def random_config(rng):
    """Hyperparameters drawn across their valid ranges (fp32 values)."""
    n_time = int(rng.integers(0, 12))
    kw = dict(beta_m=sorted(rng.uniform(0.0, 0.99, 3).tolist()), beta_v=float(rng.uniform(0.9, 0.9999)),
              beta_f=sorted(rng.uniform(0.5, 0.999, 3).tolist()), eps_v=float(10 ** rng.uniform(-10, -6)),
              eps_f=float(10 ** rng.uniform(-24, -16)), eps_norm=float(10 ** rng.uniform(-32, -20)),
              exp_mult=float(rng.uniform(1e-4, 0.1)), step_mult=float(rng.uniform(1e-4, 1e-2)),
              lr=float(rng.uniform(0.1, 2.0)), weight_decay=float(rng.uniform(0.0, 0.1)), n_time=n_time,
              timescales=sorted((10 ** rng.uniform(0, 5, n_time)).tolist()) if n_time else [],
              n_feat=int(rng.choice([L.LOPT_N_FEATURES, L.LOPT_VELO_FEATURES])))
    return kw


@pytest.mark.parametrize("case", range(24))
def test_random_shapes_and_hyperparameters(case):
    # seeded draws of tensor shapes (1-D, thin, square-ish, column counts with
    # and without 64 | cols) and of every hyperparameter, 3 steps, both MLP paths
    rng = np.random.default_rng(1000 + case)
    shapes = []
    for _ in range(5):
        k = rng.integers(0, 4)
        if k == 0:
            shapes.append((int(rng.integers(1, 5000)),))
        elif k == 1:
            shapes.append((int(rng.integers(2, 40)), 64 * int(rng.integers(1, 20))))
        else:
            shapes.append((int(rng.integers(2, 300)), int(rng.integers(1, 300))))
    kw = random_config(rng)
    if case == 5 or case % 7 == 6:
        kw["eps_v"] = 0.0   # the kernels' general 1/sqrt path (subnormal-safe)
    w = W.custom_workload(f"rand{case}", shapes, grad_std=float(10 ** rng.uniform(-4, -1)), steps=3,
                          prewarm_std=1e-3 if case % 2 else None, wid=200 + case)
    weights = W.mlp_weights(kw["n_time"], seed=(7, case), bias_std=0.1, n_feat=kw["n_feat"])
    for impl in IMPLS:
        check(parity(w, weights, L.config_from(mlp_impl=impl, **kw), torch))


def test_optimizer_state_dict_round_trip_continues_bitwise():
    # checkpoint after 3 of 6 steps through torch.save / torch.load(weights_only=True),
    # restore into a fresh optimizer over copies of the parameters, finish: the
    # result equals the uninterrupted 6 steps bit for bit
    import io
    w = W.custom_workload("ckpt", [(37, 64), (9,), (5, 300)], grad_std=1e-2, steps=6, wid=140)
    weights = mlp(bias_std=0.1)

    def params():
        return [torch.from_numpy(W.param_init(w, i).reshape(t.shape)).cuda() for i, t in enumerate(w.tensors)]

    def run(opt, ps, steps):
        for t in steps:
            for i, (p, tt) in enumerate(zip(ps, w.tensors)):
                p.grad = torch.from_numpy(W.grad_at(w, i, t).reshape(tt.shape)).cuda()
            opt.step()

    pa = params()
    a = L.LearnedOptimizer(pa, weights, lr=0.7, weight_decay=0.01)
    run(a, pa, range(1, 7))
    pb = params()
    b = L.LearnedOptimizer(pb, weights, lr=0.7, weight_decay=0.01)
    run(b, pb, range(1, 4))
    buf = io.BytesIO()
    torch.save({"params": [p.detach().cpu() for p in pb], "opt": b.state_dict()}, buf)
    buf.seek(0)
    ck = torch.load(buf, weights_only=True)
    pc = [p.cuda() for p in ck["params"]]
    c = L.LearnedOptimizer(pc, weights, lr=1.0, weight_decay=0.0)   # restored from the checkpoint
    c.load_state_dict(ck["opt"])
    assert c.lopt.t == 3 and c.param_groups[0]["lr"] == 0.7
    run(c, pc, range(4, 7))
    torch.cuda.synchronize()
    for i in range(len(w.tensors)):
        assert torch.equal(pa[i], pc[i])
        assert torch.equal(a.lopt.states[i], c.lopt.states[i])
    for o in (a, b, c):
        o.lopt.close()
