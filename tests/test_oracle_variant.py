"""Pins of the oracle's VeLO-shaped variant (n_feat = 19 per-element features
plus 11 step features: the d_feat of about 30 that the PyLO page gives VeLO in
"Use of the memory hierarchy").  Same machinery as the small_fc_lopt pins:
closed forms on a constant rank-1 gradient through selector networks, the
unit-mean-square invariant, an independent MLP implementation and the
scalar-loop twin."""

import numpy as np
import pytest

from oracle import Hyper, Mlp, VELO_FEATURES, mlp_size, pack_mlp, step, step_tensor, unpack_mlp
from oracle.scalar_twin import twin_step, unpack as twin_unpack
from oracle_helpers import random_case, rng
from test_oracle_pins import F64, f64_state, rank1, rank1_expected_inputs

NF = VELO_FEATURES
HPV0 = Hyper(eps_v=0.0, eps_f=0.0, eps_norm=0.0, n_feat=NF)


def selector(d, n_time=11):
    W1 = np.zeros((32, NF + n_time)); W1[0, d] = 1.0; W1[1, d] = -1.0
    W2 = np.zeros((32, 32)); W2[0, 0] = 1.0; W2[1, 1] = 1.0
    W3 = np.zeros((2, 32)); W3[0, 0] = 1.0; W3[0, 1] = -1.0
    return Mlp(W1, np.zeros(32), W2, np.zeros(32), W3, np.zeros(2))


def random_mlp_v(seed, n_time=11, bias_std=0.1):
    r = rng(20_000 + seed)
    d_in = NF + n_time
    m = Mlp(r.standard_normal((32, d_in)) / np.sqrt(d_in), r.standard_normal(32) * bias_std,
            r.standard_normal((32, 32)) / np.sqrt(32), r.standard_normal(32) * bias_std,
            r.standard_normal((2, 32)) / np.sqrt(32), r.standard_normal(2) * bias_std)
    return unpack_mlp(pack_mlp(m), n_time, NF)


def test_mlp_has_30_inputs():
    assert mlp_size(11, NF) == 32 * 30 + 32 + 32 * 32 + 32 + 2 * 32 + 2 == 2114
    assert mlp_size(0, NF) == 32 * 19 + 32 + 32 * 32 + 32 + 2 * 32 + 2


@pytest.mark.parametrize("d", list(range(NF + 11)))
def test_each_input_matches_rank1_closed_form(d):
    # input d < 19 is the normalised feature F_d; input 19 + q is tanh(t / tau_q)
    R, C, T = 5, 7, 3
    alpha, beta, g = rank1(R, C, seed=60)
    p = rng(61).standard_normal((R, C)) * 0.02
    st = f64_state(R, C)
    sel = selector(d)
    for s in range(1, T):
        p, st, _ = step_tensor(p, g, st, s, sel, HPV0, store_dtype=F64)
    p_last = p.copy()
    _, _, info = step_tensor(p, g, st, T, sel, HPV0, keep=True, store_dtype=F64)
    _, x = rank1_expected_inputs(alpha, beta, p_last, T, HPV0)
    expect = x[d] if d < NF else x[28 + (d - NF)]
    assert info.x.shape[-1] == NF + 11
    np.testing.assert_allclose(info.u / HPV0.step_mult, expect, rtol=1e-11, atol=1e-13)


@pytest.mark.parametrize("shape", [(6, 11), (1, 40), (9, 1)])
def test_normalised_features_have_unit_mean_square(shape):
    p, g, st = random_case(*shape, seed=62)
    _, _, info = step_tensor(p, g, st, 3, random_mlp_v(1), Hyper(n_feat=NF), keep=True)
    xs = info.x[..., :NF]
    np.testing.assert_allclose(np.mean(xs * xs, axis=(0, 1)), np.ones(NF), rtol=1e-12)


def test_mlp_matches_torch_sequential():
    torch = pytest.importorskip("torch")
    w = random_mlp_v(2)
    seq = torch.nn.Sequential(torch.nn.Linear(30, 32), torch.nn.ReLU(), torch.nn.Linear(32, 32),
                              torch.nn.ReLU(), torch.nn.Linear(32, 2)).double()
    with torch.no_grad():
        for lin, W, b in ((seq[0], w.W1, w.b1), (seq[2], w.W2, w.b2), (seq[4], w.W3, w.b3)):
            lin.weight.copy_(torch.from_numpy(W)); lin.bias.copy_(torch.from_numpy(b))
    p, g, st = random_case(4, 9, seed=63)
    hp = Hyper(step_mult=1.0, exp_mult=0.5, n_feat=NF)
    _, _, info = step_tensor(p, g, st, 2, w, hp, keep=True)
    out = seq(torch.from_numpy(info.x.reshape(-1, 30))).detach().numpy()
    np.testing.assert_allclose(info.u.ravel(), out[:, 0] * np.exp(out[:, 1] * 0.5), rtol=1e-12, atol=1e-15)


@pytest.mark.parametrize("R,C", [(4, 4), (1, 4), (4, 1), (3, 5), (1, 1)])
def test_scalar_twin_agrees_ten_steps(R, C):
    # as P10: the fp64 update and accumulators to 1e-12, the stored fp32 values
    # to one rounding, stepping both from the same fp32 state
    flat = pack_mlp(random_mlp_v(3))
    hp = Hyper(n_feat=NF).as_f32()
    mlp = unpack_mlp(flat, 11, NF)
    w = twin_unpack(flat, 11, NF)
    p, _, st = random_case(R, C, seed=64)
    for t in range(1, 11):
        g = random_case(R, C, seed=640 + t)[1]
        pn, sn, info = step_tensor(p, g, st, t, mlp, hp, keep=True)
        tp, _, raw = twin_step(p.astype(float).tolist(), g.astype(float).tolist(),
                               {k: v.astype(float).tolist() for k, v in st.items()}, t, w, hp)
        np.testing.assert_allclose(np.array(raw["u"]), info.u, rtol=1e-12, atol=1e-18)
        for k in ("m", "v", "r", "c"):
            np.testing.assert_allclose(np.array(raw[k]), getattr(info.acc, k), rtol=1e-13, atol=1e-300)
        np.testing.assert_allclose(np.array(tp, np.float32), pn, rtol=1.5e-7, atol=1e-30)
        p, st = pn, sn


def test_variant_ignores_the_cross_features():
    # The variant equals small_fc_lopt with W1's nine m_a rho_k columns set to
    # zero: the other features and their normalisation do not depend on them.
    p, g, st = random_case(5, 6, seed=65)
    wv = random_mlp_v(4)
    W1f = np.zeros((32, 39))
    W1f[:, :NF] = wv.W1[:, :NF]
    W1f[:, 28:] = wv.W1[:, NF:]
    wf = Mlp(W1f, wv.b1, wv.W2, wv.b2, wv.W3, wv.b3)
    pv, sv, iv = step_tensor(p, g, st, 4, wv, Hyper(n_feat=NF), keep=True)
    pf, sf, if_ = step_tensor(p, g, st, 4, wf, Hyper(), keep=True)
    np.testing.assert_allclose(iv.u, if_.u, rtol=1e-12, atol=1e-18)
    np.testing.assert_array_equal(pv, pf)


def test_unknown_feature_count_is_rejected():
    flat = np.zeros(mlp_size(11, 20), np.float32)
    p, g, st = random_case(2, 2, seed=66)
    with pytest.raises(ValueError):
        step([p], [g], [st], 1, flat, Hyper(n_feat=20))
