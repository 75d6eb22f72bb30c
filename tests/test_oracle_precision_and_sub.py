"""Pins of two oracle pieces that the other pins leave open.

* ``Hyper.as_f32``: the hyperparameters reach the library as fp32 numbers
  (reading R25), so the oracle rounds every real-valued field to fp32 before
  use.  A field the rounding missed would only show up against the GPU; here
  every float field of the dataclass is set to a value that fp32 cannot hold
  and must come back as its fp32 rounding.  The moving averages after one
  step from zero state then follow their closed forms with the fp32 decays:
  m_a = (1 - fl32(beta_a)) g, v = (1 - fl32(beta_v)) g^2,
  r_k = (1 - fl32(beta_k)) (mean_j g^2 + fl32(eps_f)), which differ from the
  fp64-decay forms by ~1e-5 relative (fl32(0.999) moves 1 - beta_v by 1.3e-5),
  the size of the parity bar.
* ``step_tensor_sub``: the update evaluated on a sub-block of rows and columns
  equals the whole-tensor step at those positions, and its per-tensor
  statistics (feature scales, row/column averages) are those of the whole
  tensor: each row or column index mix-up (the column averages of the wrong
  columns, the row term of the wrong rows, statistics over the sub-block only)
  moves the result far beyond rounding.
"""
import dataclasses

import numpy as np
import pytest

from oracle import Hyper, Mlp, step, step_tensor, step_tensor_sub, zero_state
from oracle_helpers import random_case, random_mlp, rng


def f32(x):
    return float(np.float32(x))


def unrepresentable(k):
    """A value near 0.1 * (k + 1) that fp32 cannot hold exactly."""
    x = 0.1 * (k + 1) + 1e-9 * (k + 1)
    assert f32(x) != x
    return x


def test_as_f32_rounds_every_real_field():
    fields = dataclasses.fields(Hyper)
    kw, k = {}, 0
    for f in fields:
        v = getattr(Hyper(), f.name)
        if isinstance(v, float):
            kw[f.name] = unrepresentable(k)
            k += 1
        elif isinstance(v, tuple):
            kw[f.name] = tuple(unrepresentable(k + j) for j in range(len(v)))
            k += len(v)
    hp = Hyper(**kw)
    h32 = hp.as_f32()
    assert {f.name for f in dataclasses.fields(h32)} == {f.name for f in fields}
    checked = 0
    for f in fields:
        a, b = getattr(hp, f.name), getattr(h32, f.name)
        if isinstance(a, float):
            assert b == f32(a) and b != a, f.name
            checked += 1
        elif isinstance(a, tuple):
            if f.name == "timescales":
                a = a[: hp.n_time]
            assert len(b) == len(a), f.name
            for x, y in zip(a, b):
                assert y == f32(x) and y != x, f.name
            checked += 1
        else:
            assert a == b, f.name
    # beta_m, beta_v, beta_f, eps_v, eps_f, eps_norm, exp_mult, step_mult, lr,
    # weight_decay, timescales
    assert checked == 11


def test_one_step_accumulators_follow_the_closed_forms_with_fp32_decays():
    R, C = 9, 14
    g = (rng(77).standard_normal((R, C)) * 1e-2).astype(np.float32)
    p = np.zeros((R, C), np.float32)
    hp = Hyper()
    _, [st] = step([p], [g], [zero_state(R, C)], 1, np.zeros(2402, np.float32), hp)
    g64 = g.astype(np.float64)
    for a in range(3):
        want = ((1.0 - f32(hp.beta_m[a])) * g64).astype(np.float32)
        assert np.array_equal(st["m"][a], want)
    v_want = ((1.0 - f32(hp.beta_v)) * g64 * g64).astype(np.float32)
    v_f64_decay = ((1.0 - hp.beta_v) * g64 * g64).astype(np.float32)
    assert np.array_equal(st["v"], v_want)
    assert np.mean(st["v"] != v_f64_decay) > 0.9      # the fp32 decay is what makes the difference
    row_mean = (g64 * g64).mean(axis=1)
    col_mean = (g64 * g64).mean(axis=0)
    for k in range(3):
        ob = 1.0 - f32(hp.beta_f[k])
        np.testing.assert_array_equal(st["r"][k], (ob * (row_mean + f32(hp.eps_f))).astype(np.float32))
        np.testing.assert_array_equal(st["c"][k], (ob * (col_mean + f32(hp.eps_f))).astype(np.float32))


@pytest.mark.parametrize("shape,rows,cols", [
    ((40, 70), [0, 3, 17, 39], None),
    ((40, 70), None, [0, 1, 33, 69]),
    ((40, 70), [5, 6, 38], [2, 40, 41, 68]),
    ((1, 5000), None, [0, 1, 2, 777, 4097, 4999]),
    ((300, 1), [0, 150, 299], None),
])
@pytest.mark.parametrize("n_feat", [28, 19])
def test_sub_block_step_equals_the_whole_step_there(shape, rows, cols, n_feat):
    R, C = shape
    p, g, st = random_case(R, C, seed=31)
    hp = Hyper(n_feat=n_feat, lr=0.7, weight_decay=0.01).as_f32()
    mlp = random_mlp(5)
    if n_feat == 19:
        mlp = Mlp(np.concatenate([mlp.W1[:, :19], mlp.W1[:, 28:]], axis=1), mlp.b1, mlp.W2, mlp.b2, mlp.W3, mlp.b3)
    p_full, st_full, info_full = step_tensor(p, g, st, 4, mlp, hp, keep=True)
    p_sub, st_sub, info_sub = step_tensor_sub(p, g, st, 4, mlp, hp, rows, cols)
    ri = np.arange(R) if rows is None else np.asarray(rows)
    ci = np.arange(C) if cols is None else np.asarray(cols)
    np.testing.assert_allclose(p_sub, p_full.reshape(R, C)[np.ix_(ri, ci)], rtol=2e-7, atol=0)
    np.testing.assert_array_equal(st_sub["m"], st_full["m"][:, ri][:, :, ci])
    np.testing.assert_array_equal(st_sub["v"], st_full["v"][np.ix_(ri, ci)])
    np.testing.assert_array_equal(st_sub["r"], st_full["r"])
    np.testing.assert_array_equal(st_sub["c"], st_full["c"])
    np.testing.assert_array_equal(info_sub.scales, info_full.scales)
    np.testing.assert_array_equal(info_sub.acc.rbar, info_full.acc.rbar)
    # and the update does depend on the sub-block's own rows and columns
    assert not np.allclose(p_sub, p.reshape(R, C)[np.ix_(ri, ci)], rtol=1e-9, atol=0)
