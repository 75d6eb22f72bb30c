"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each test names what it pins.  Expected values come from closed forms of the
recurrences, invariants of the normalisation, degenerate shapes, a scalar-loop
brute force, or an independent library MLP; none retypes the oracle's code.
"""
import math

import numpy as np
import pytest

from oracle import (Hyper, Mlp, accumulate, cross_index, pack_mlp, step, step_tensor,
                    zero_state)
from oracle_helpers import magnitude_selector_mlp, random_case, random_mlp, rng, selector_mlp

HP0 = Hyper(eps_v=0.0, eps_f=0.0, eps_norm=0.0)   # epsilon-free: closed forms are exact
F64 = np.float64


def run(p, grads, st, hp, mlp, t0=1, keep_last=True, store=F64):
    """Run len(grads) steps from state st; returns p, state, info of the last step."""
    info = None
    for s, g in enumerate(grads):
        last = s == len(grads) - 1
        p, st, info = step_tensor(p, g, st, t0 + s, mlp, hp, keep=keep_last and last,
                                  store_dtype=store)
    return p, st, info


def f64_state(R, C):
    return {k: v.astype(F64) for k, v in zero_state(R, C).items()}


def rank1(R, C, seed):
    r = rng(seed)
    alpha = r.uniform(0.5, 1.5, R) * r.choice([-1.0, 1.0], R)
    beta = r.uniform(0.5, 1.5, C) * r.choice([-1.0, 1.0], C)
    return alpha, beta, np.outer(alpha, beta)


# --------------------------------------------------------------- P1 normalisation
@pytest.mark.parametrize("shape", [(7, 13), (1, 33), (16, 1), (5, 5)])
def test_p1_normalised_features_have_unit_mean_square(shape):
    p, g, st = random_case(*shape, seed=1)
    _, _, info = step_tensor(p, g, st, 3, random_mlp(1), Hyper(), keep=True)
    xhat = info.x[..., :28]
    ms = (xhat ** 2).reshape(-1, 28).mean(axis=0)
    np.testing.assert_allclose(ms, 1.0, rtol=0, atol=1e-12)
    # and normalisation is a pure per-feature scaling of the raw features
    ratio = xhat / info.F
    np.testing.assert_allclose(ratio, np.broadcast_to(ratio[:1, :1], ratio.shape), rtol=1e-12)


# --------------------------------------------------------------- P2/P3 update formula
def test_p2_zero_output_layer_leaves_params_bitwise():
    p, g, st = random_case(6, 9, seed=2)
    m = random_mlp(2)
    m0 = Mlp(m.W1, m.b1, m.W2, m.b2, np.zeros((2, 32)), np.zeros(2))
    p_new, st_new, _ = step_tensor(p, g, st, 1, m0, Hyper())
    assert p_new.dtype == np.float32 and np.array_equal(p_new, p)
    for k in ("m", "v", "r", "c"):
        assert not np.array_equal(st_new[k], st[k]), k   # accumulators still advance


@pytest.mark.parametrize("c0,c1", [(0.7, -2.0), (-1.3, 5.0), (2.0, 0.0)])
def test_p3_constant_output_gives_closed_form_update(c0, c1):
    p, g, st = random_case(4, 7, seed=3)
    m = random_mlp(3)
    mc = Mlp(m.W1, m.b1, m.W2, m.b2, np.zeros((2, 32)), np.array([c0, c1]))
    hp = Hyper(exp_mult=0.25, step_mult=0.01)
    _, _, info = step_tensor(p, g, st, 1, mc, hp, keep=True)
    expected = c0 * math.exp(c1 * 0.25) * 0.01
    np.testing.assert_allclose(info.u, expected, rtol=1e-15)


def test_p3b_lr_and_decoupled_weight_decay():
    p, g, st = random_case(3, 4, seed=4)
    m = random_mlp(4)
    mc = Mlp(m.W1, m.b1, m.W2, m.b2, np.zeros((2, 32)), np.array([0.5, 0.0]))
    hp = Hyper(step_mult=0.01, lr=0.5, weight_decay=0.1)
    p_new, _, _ = step_tensor(p, g, st, 1, mc, hp, store_dtype=F64)
    # u = 0.5 * 0.01 everywhere; p <- p - lr*u - lr*wd*p
    np.testing.assert_allclose(p_new, p.astype(F64) * (1 - 0.05) - 0.5 * 0.005, rtol=1e-14)


def test_p3c_per_tensor_lr_and_weight_decay():
    # constant output dir = 0.5, mag = 0: u = 0.5 step_mult everywhere; with
    # per-tensor (lr_i, wd_i) tensor i gets exactly p (1 - lr_i wd_i) - lr_i u,
    # whatever the list-wide lr and wd say (all values exact in fp32)
    cases = [random_case(3, 4, seed=40), random_case(1, 6, seed=41), random_case(5, 1, seed=42)]
    m = random_mlp(4)
    mc = Mlp(m.W1, m.b1, m.W2, m.b2, np.zeros((2, 32)), np.array([0.5, 0.0]))
    hp = Hyper(step_mult=2.0 ** -7, lr=8.0, weight_decay=4.0)
    th = [(0.5, 0.125), (2.0, 0.0), (0.25, 0.375)]
    ps, _ = step([c[0] for c in cases], [c[1] for c in cases], [c[2] for c in cases], 1, pack_mlp(mc), hp,
                 tensor_hyper=th, store_dtype=F64)
    for (p, _, _), (lr, wd), p_new in zip(cases, th, ps):
        np.testing.assert_allclose(p_new, p.astype(F64) * (1 - lr * wd) - lr * 0.5 * 2.0 ** -7, rtol=1e-14)
    with pytest.raises(ValueError):
        step([c[0] for c in cases], [c[1] for c in cases], [c[2] for c in cases], 1, pack_mlp(mc), hp,
             tensor_hyper=th[:2])


def test_p3d_tensor_without_gradient_is_left_as_is():
    # R28: a None gradient leaves its tensor and state untouched, and the other
    # tensors step exactly as they would without it in the list
    cases = [random_case(4, 6, seed=43), random_case(1, 9, seed=44), random_case(3, 3, seed=45)]
    w = pack_mlp(random_mlp(5))
    ps, sts = step([c[0] for c in cases], [cases[0][1], None, cases[2][1]], [c[2] for c in cases], 2, w, Hyper())
    assert ps[1] is cases[1][0] and sts[1] is cases[1][2]
    ref_p, ref_s = step([cases[0][0], cases[2][0]], [cases[0][1], cases[2][1]], [cases[0][2], cases[2][2]], 2, w,
                        Hyper())
    for a, b in ((0, 0), (2, 1)):
        assert np.array_equal(ps[a], ref_p[b])
        for k in ("m", "v", "r", "c"):
            assert np.array_equal(sts[a][k], ref_s[b][k])


# --------------------------------------------------------------- P4 features via selectors
def rank1_expected_inputs(alpha, beta, p_last, t, hp):
    """Closed-form MLP inputs after t steps of the constant rank-1 gradient alpha beta^T
    from zero state, with all epsilons zero.

    m_a = (1 - b_a^t) g, v = (1 - b_v^t) g^2, r_k[i] = (1 - f_k^t) alpha_i^2 mean(beta^2),
    c_k[j] = (1 - f_k^t) beta_j^2 mean(alpha^2), so r c / rbar = (1 - f_k^t) g^2.
    Each feature is then a known function of (alpha, beta, p); the MLP sees it
    divided by its root-mean-square over the tensor.
    """
    g = np.outer(alpha, beta)
    R, C = g.shape
    sg = np.sign(g)
    one = np.ones_like(g)
    dv = 1 - hp.beta_v ** t
    raw = {0: g, 1: p_last, 5: dv * g * g, 9: 1.0 / (math.sqrt(dv) * np.abs(g))}
    for a in range(3):
        raw[2 + a] = (1 - hp.beta_m[a] ** t) * g
        raw[6 + a] = (1 - hp.beta_m[a] ** t) / math.sqrt(1 - hp.beta_v ** t) * sg
    for k in range(3):
        dk = 1 - hp.beta_f[k] ** t
        raw[10 + k] = sg / math.sqrt(dk)
        raw[13 + k] = (1.0 / np.abs(alpha))[:, None] * one / math.sqrt(dk * np.mean(beta ** 2))
        raw[16 + k] = (1.0 / np.abs(beta))[None, :] * one / math.sqrt(dk * np.mean(alpha ** 2))
        for a in range(3):
            raw[cross_index(a, k)] = (1 - hp.beta_m[a] ** t) / math.sqrt(dk) * sg
    x = {d: f / np.sqrt(np.mean(f * f)) for d, f in raw.items()}
    for q in range(hp.n_time):
        x[28 + q] = np.tanh(t / hp.timescales[q]) * one
    return raw, x


@pytest.mark.parametrize("d", list(range(39)))
def test_p4_each_mlp_input_matches_rank1_closed_form(d):
    R, C, T = 5, 7, 4
    alpha, beta, g = rank1(R, C, seed=40)
    p0 = (rng(41).standard_normal((R, C)) * 0.02)
    sel = selector_mlp(d)
    p = p0.copy()
    st = f64_state(R, C)
    for s in range(1, T):
        p, st, _ = step_tensor(p, g, st, s, sel, HP0, store_dtype=F64)
    p_last = p.copy()
    _, _, info = step_tensor(p, g, st, T, sel, HP0, keep=True, store_dtype=F64)
    _, x = rank1_expected_inputs(alpha, beta, p_last, T, HP0)
    # dir = relu(x_d) - relu(-x_d) = x_d, mag = 0  ->  u = step_mult * x_d
    np.testing.assert_allclose(info.u / HP0.step_mult, x[d], rtol=1e-11, atol=1e-13)


@pytest.mark.parametrize("d", [0, 5, 12, 17, 27, 30])
def test_p5_magnitude_channel(d):
    R, C, T = 4, 6, 2
    alpha, beta, g = rank1(R, C, seed=50)
    p = rng(51).standard_normal((R, C)) * 0.02
    hp = Hyper(eps_v=0.0, eps_f=0.0, eps_norm=0.0, exp_mult=0.3, step_mult=0.01)
    sel = magnitude_selector_mlp(d)
    st = f64_state(R, C)
    p1, st, _ = step_tensor(p, g, st, 1, sel, hp, store_dtype=F64)
    _, _, info = step_tensor(p1, g, st, 2, sel, hp, keep=True, store_dtype=F64)
    _, x = rank1_expected_inputs(alpha, beta, p1, T, hp)
    np.testing.assert_allclose(info.u, np.exp(0.3 * x[d]) * 0.01, rtol=1e-12)


def test_p4b_hidden_biases_enter_before_relu():
    # W1 = 0, b1 = beta, W2 = I, b2 = gamma, W3 row 0 = e_o  ->  dir = relu(relu(beta_o) + gamma_o)
    p, g, st = random_case(3, 3, seed=6)
    b1 = np.linspace(-1, 1, 32)
    b2 = np.linspace(0.5, -0.5, 32)
    for o in (0, 3, 16, 31):
        W3 = np.zeros((2, 32)); W3[0, o] = 1.0
        m = Mlp(np.zeros((32, 39)), b1, np.eye(32), b2, W3, np.zeros(2))
        _, _, info = step_tensor(p, g, st, 1, m, Hyper(step_mult=1.0), keep=True)
        np.testing.assert_allclose(info.u, max(max(b1[o], 0.0) + b2[o], 0.0), rtol=1e-15)


def test_p4c_mlp_matches_torch_sequential():
    torch = pytest.importorskip("torch")
    w = random_mlp(7)
    seq = torch.nn.Sequential(torch.nn.Linear(39, 32), torch.nn.ReLU(), torch.nn.Linear(32, 32),
                              torch.nn.ReLU(), torch.nn.Linear(32, 2)).double()
    with torch.no_grad():
        for lin, W, b in ((seq[0], w.W1, w.b1), (seq[2], w.W2, w.b2), (seq[4], w.W3, w.b3)):
            lin.weight.copy_(torch.from_numpy(W)); lin.bias.copy_(torch.from_numpy(b))
    p, g, st = random_case(5, 6, seed=7)
    hp = Hyper(step_mult=1.0, exp_mult=0.5)
    _, _, info = step_tensor(p, g, st, 2, w, hp, keep=True)
    out = seq(torch.from_numpy(info.x.reshape(-1, 39))).detach().numpy()
    expect = out[:, 0] * np.exp(out[:, 1] * 0.5)
    np.testing.assert_allclose(info.u.ravel(), expect, rtol=1e-12, atol=1e-15)


def test_p4d_time_features_start_at_t1_and_zero_features_are_finite():
    # t is 1-based: the first step sees tanh(1 / 1), not tanh(0)
    R, C = 2, 3
    p = np.zeros((R, C), np.float32)
    g = np.zeros((R, C), np.float32)
    _, _, info = step_tensor(p, g, zero_state(R, C), 1, selector_mlp(28), Hyper(step_mult=1.0), keep=True)
    np.testing.assert_allclose(info.u, math.tanh(1.0), rtol=1e-15)
    # with all-zero gradients and parameters every input is finite
    assert np.all(np.isfinite(info.x))


def test_n_time_zero_has_28_inputs():
    R, C = 3, 4
    alpha, beta, g = rank1(R, C, seed=8)
    p = rng(9).standard_normal((R, C)) * 0.02
    hp = Hyper(eps_v=0.0, eps_f=0.0, eps_norm=0.0, n_time=0)
    for d in (0, 13, 27):
        _, _, info = step_tensor(p, g, f64_state(R, C), 1, selector_mlp(d, n_time=0), hp,
                                 keep=True, store_dtype=F64)
        _, x = rank1_expected_inputs(alpha, beta, p, 1, hp)
        assert info.x.shape[-1] == 28
        np.testing.assert_allclose(info.u / hp.step_mult, x[d], rtol=1e-11, atol=1e-13)


# --------------------------------------------------------------- P6 EMA closed forms
def test_p6_ema_closed_forms_constant_gradient():
    R, C, K = 4, 5, 9
    g = rng(60).standard_normal((R, C))
    hp = Hyper()
    st = f64_state(R, C)
    for _ in range(K):
        acc = accumulate(g, st, hp)
        st = {"m": acc.m, "v": acc.v, "r": acc.r, "c": acc.c}
    for a in range(3):
        np.testing.assert_allclose(acc.m[a], (1 - hp.beta_m[a] ** K) * g, rtol=1e-13)
    np.testing.assert_allclose(acc.v, (1 - hp.beta_v ** K) * g * g, rtol=1e-12)
    gr = (g * g).mean(axis=1)
    gc = (g * g).mean(axis=0)
    for k in range(3):
        np.testing.assert_allclose(acc.r[k], (1 - hp.beta_f[k] ** K) * (gr + hp.eps_f), rtol=1e-12)
        np.testing.assert_allclose(acc.c[k], (1 - hp.beta_f[k] ** K) * (gc + hp.eps_f), rtol=1e-12)
        np.testing.assert_allclose(acc.rbar[k], (1 - hp.beta_f[k] ** K) * (gr.mean() + hp.eps_f),
                                   rtol=1e-12)


def test_p6_ema_weighted_sum_varying_gradient():
    R, C, K = 3, 4, 6
    gs = [rng(61 + s).standard_normal((R, C)) for s in range(K)]
    hp = Hyper()
    st = f64_state(R, C)
    for g in gs:
        acc = accumulate(g, st, hp)
        st = {"m": acc.m, "v": acc.v, "r": acc.r, "c": acc.c}
    for a in range(3):
        b = hp.beta_m[a]
        want = sum((1 - b) * b ** (K - 1 - s) * gs[s] for s in range(K))
        np.testing.assert_allclose(acc.m[a], want, rtol=1e-12, atol=1e-300)
    bv = hp.beta_v
    np.testing.assert_allclose(acc.v, sum((1 - bv) * bv ** (K - 1 - s) * gs[s] ** 2 for s in range(K)),
                               rtol=1e-12)
    for k in range(3):
        f = hp.beta_f[k]
        want_c = sum((1 - f) * f ** (K - 1 - s) * ((gs[s] ** 2).mean(axis=0) + hp.eps_f) for s in range(K))
        np.testing.assert_allclose(acc.c[k], want_c, rtol=1e-12)


# --------------------------------------------------------------- P7 factored reconstruction
def test_p7_rank1_factored_features_exact():
    R, C, T = 6, 4, 5
    alpha, beta, g = rank1(R, C, seed=70)
    p = rng(71).standard_normal((R, C)) * 0.02
    st = f64_state(R, C)
    for s in range(1, T + 1):
        pn, st, info = step_tensor(p, g, st, s, random_mlp(7), HP0, keep=True, store_dtype=F64)
        raw, _ = rank1_expected_inputs(alpha, beta, p, s, HP0)
        for d in range(28):
            np.testing.assert_allclose(info.F[..., d], raw[d], rtol=1e-12, err_msg=f"feature {d} step {s}")
        p = pn


# --------------------------------------------------------------- P8/P9 degenerate shapes
def test_p8_vector_is_unfactored():
    n, T = 11, 3
    r = rng(80)
    g = r.uniform(0.5, 1.5, n) * r.choice([-1.0, 1.0], n)
    p = r.standard_normal(n) * 0.02
    st = f64_state(1, n)
    for s in range(1, T + 1):
        p, st, info = step_tensor(p, g, st, s, random_mlp(8), HP0, keep=True, store_dtype=F64)
    for k in range(3):
        dk = 1 - HP0.beta_f[k] ** T
        # per-element column accumulator: c_k = (1 - f^t) g^2, rho_k = c_k^(-1/2)
        np.testing.assert_allclose(st["c"][k], dk * g * g, rtol=1e-13)
        np.testing.assert_allclose(info.F[0, :, 10 + k], np.sign(g) / math.sqrt(dk), rtol=1e-12)
        np.testing.assert_allclose(info.x[0, :, 13 + k], 1.0, rtol=1e-14)   # constant row feature


def test_p9_single_element_features_are_signs():
    p, g, st = random_case(1, 1, seed=9)
    _, _, info = step_tensor(p, g, st, 4, random_mlp(9), Hyper(), keep=True)
    np.testing.assert_allclose(info.x[0, 0, :28], np.sign(info.F[0, 0, :]), rtol=1e-14)
    # through the selector network too
    for d in (0, 1, 9, 22):
        _, _, inf2 = step_tensor(p, g, st, 4, selector_mlp(d), Hyper(step_mult=1.0), keep=True)
        assert abs(abs(inf2.u[0, 0]) - 1.0) < 1e-14


# --------------------------------------------------------------- P11-P14 symmetries
def test_p11_row_column_permutation_equivariance():
    p, g, st = random_case(5, 8, seed=11)
    pr = rng(111).permutation(5)
    pc = rng(112).permutation(8)
    w = random_mlp(11)
    _, st1, i1 = step_tensor(p, g, st, 2, w, Hyper(), keep=True)
    stp = {"m": st["m"][:, pr][:, :, pc], "v": st["v"][pr][:, pc], "r": st["r"][:, pr], "c": st["c"][:, pc]}
    _, st2, i2 = step_tensor(p[pr][:, pc], g[pr][:, pc], stp, 2, w, Hyper(), keep=True)
    np.testing.assert_allclose(i2.u, i1.u[pr][:, pc], rtol=1e-11)
    np.testing.assert_array_equal(st2["r"], st1["r"][:, pr])
    np.testing.assert_array_equal(st2["c"], st1["c"][:, pc])


def test_p12_transpose_symmetry():
    # transposing swaps the row and column accumulators; with W1 columns 13-15 <-> 16-18
    # exchanged, the update is the transposed one (rbar only rescales rho, which the
    # normalisation removes).
    p, g, st = random_case(4, 9, seed=12)
    w = random_mlp(12)
    W1s = w.W1.copy()
    W1s[:, 13:16], W1s[:, 16:19] = w.W1[:, 16:19], w.W1[:, 13:16]
    ws = Mlp(W1s, w.b1, w.W2, w.b2, w.W3, w.b3)
    _, s1, i1 = step_tensor(p, g, st, 3, w, Hyper(), keep=True)
    stT = {"m": st["m"].transpose(0, 2, 1), "v": st["v"].T, "r": st["c"], "c": st["r"]}
    _, s2, i2 = step_tensor(p.T, g.T, stT, 3, ws, Hyper(), keep=True)
    np.testing.assert_allclose(i2.u, i1.u.T, rtol=1e-10)
    np.testing.assert_array_equal(s2["r"], s1["c"])


@pytest.mark.parametrize("s,exact", [(4.0, True), (3.0, False)])
def test_p13_gradient_scale_invariance_without_epsilons(s, exact):
    p, g, st = random_case(5, 6, seed=13)
    w = random_mlp(13)
    st64 = {k: v.astype(F64) for k, v in st.items()}
    sst = {"m": st64["m"] * s, "v": st64["v"] * s * s, "r": st64["r"] * s * s, "c": st64["c"] * s * s}
    _, _, i1 = step_tensor(p, g.astype(F64), st64, 2, w, HP0, keep=True, store_dtype=F64)
    _, _, i2 = step_tensor(p, g.astype(F64) * s, sst, 2, w, HP0, keep=True, store_dtype=F64)
    if exact:
        np.testing.assert_array_equal(i1.u, i2.u)
    else:
        np.testing.assert_allclose(i1.u, i2.u, rtol=1e-12)


def test_p14_tensor_independence():
    a = random_case(3, 4, seed=14)
    b = random_case(1, 7, seed=15)
    w = pack_mlp(random_mlp(14))
    pa, sa = step([a[0]], [a[1]], [a[2]], 2, w)
    pb, sb = step([b[0]], [b[1]], [b[2]], 2, w)
    pab, sab = step([a[0], b[0]], [a[1], b[1]], [a[2], b[2]], 2, w)
    assert np.array_equal(pab[0], pa[0]) and np.array_equal(pab[1], pb[0])
    for k in ("m", "v", "r", "c"):
        assert np.array_equal(sab[0][k], sa[0][k]) and np.array_equal(sab[1][k], sb[0][k])


def test_p15_resume_equals_uninterrupted():
    p0, _, _ = random_case(4, 4, seed=16)
    gs = [random_case(4, 4, seed=160 + s)[1] for s in range(10)]
    w = pack_mlp(random_mlp(16))
    p, st = [p0], [zero_state(4, 4)]
    for t in range(1, 11):
        p, st = step(p, [gs[t - 1]], st, t, w)
    q, sq = [p0], [zero_state(4, 4)]
    for t in range(1, 6):
        q, sq = step(q, [gs[t - 1]], sq, t, w)
    saved = (q[0].copy(), {k: v.copy() for k, v in sq[0].items()}, 5)
    q, sq, t0 = [saved[0]], [saved[1]], saved[2]
    for t in range(t0 + 1, 11):
        q, sq = step(q, [gs[t - 1]], sq, t, w)
    assert np.array_equal(p[0], q[0])


def test_block_rows_only_changes_summation_order():
    p, g, st = random_case(37, 11, seed=17)
    w = random_mlp(17)
    a = step_tensor(p, g, st, 2, w, Hyper(), store_dtype=F64)
    b = step_tensor(p, g, st, 2, w, Hyper(), block_rows=5, store_dtype=F64)
    np.testing.assert_allclose(a[0], b[0], rtol=1e-14)
    np.testing.assert_allclose(a[2].sum_sq, b[2].sum_sq, rtol=1e-13)


def test_sampled_rows_equal_full_step():
    p, g, st = random_case(23, 9, seed=18)
    w = random_mlp(18)
    pf, sf, _ = step_tensor(p, g, st, 3, w, Hyper())
    rows = [0, 5, 22, 7]
    from oracle import step_tensor_rows
    pr, sr = step_tensor_rows(p, g, st, 3, w, Hyper(), rows, block_rows=4)
    np.testing.assert_allclose(pr, pf[rows], rtol=1e-7, atol=1e-30)
    np.testing.assert_array_equal(sr["r"], sf["r"])
    np.testing.assert_array_equal(sr["c"], sf["c"])
    np.testing.assert_array_equal(sr["m"], sf["m"][:, rows])
