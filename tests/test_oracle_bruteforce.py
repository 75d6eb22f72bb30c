"""P10: the vectorised oracle against the scalar-loop twin on tiny tensors.

The twin (pure Python, one element at a time) and the NumPy oracle are
compared step by step from a common fp32 state: the fp64 update and
accumulators must agree to 1e-12 relative, and the fp32 state they store must
agree to one fp32 rounding.
"""
import numpy as np
import pytest
from hypothesis import given, settings, strategies as st_

from oracle import Hyper, pack_mlp, step_tensor, unpack_mlp
from oracle.scalar_twin import twin_step, unpack
from oracle_helpers import random_case, random_mlp


def to_lists(st):
    return {"m": st["m"].astype(float).tolist(), "v": st["v"].astype(float).tolist(),
            "r": st["r"].astype(float).tolist(), "c": st["c"].astype(float).tolist()}


def compare_one_step(p, g, st, t, flat, hp):
    hp32 = hp.as_f32()
    mlp = unpack_mlp(flat, hp32.n_time)
    pn, sn, info = step_tensor(p, g, st, t, mlp, hp32, keep=True)
    tp, tst, raw = twin_step(p.astype(float).tolist(), g.astype(float).tolist(), to_lists(st), t,
                             unpack(flat, hp32.n_time), hp32)
    np.testing.assert_allclose(np.array(raw["u"]), info.u, rtol=1e-12, atol=1e-18)
    for k in ("m", "v", "r", "c"):
        np.testing.assert_allclose(np.array(raw[k]), getattr(info.acc, k), rtol=1e-13, atol=1e-300)
    np.testing.assert_allclose(np.array(tp, np.float32), pn, rtol=1.5e-7, atol=1e-30)
    return pn, sn


@pytest.mark.parametrize("shape", [(4, 4), (1, 4), (4, 1), (3, 5), (1, 1), (2, 3)])
@pytest.mark.parametrize("warm", [False, True])
def test_p10_bruteforce_ten_steps(shape, warm):
    R, C = shape
    p, _, st = random_case(R, C, seed=100 + R * 10 + C, warm=warm)
    flat = pack_mlp(random_mlp(100, bias_std=0.2))
    for t in range(1, 11):
        g = random_case(R, C, seed=1000 + t)[1]
        p, st = compare_one_step(p, g, st, t, flat, Hyper())


def test_p10_bruteforce_no_time_features_and_lr_wd():
    p, g, st = random_case(3, 4, seed=101)
    flat = pack_mlp(random_mlp(101, n_time=0))
    compare_one_step(p, g, st, 2, flat, Hyper(n_time=0, lr=0.7, weight_decay=0.05))


@settings(max_examples=25, deadline=None, derandomize=True)
@given(R=st_.integers(1, 9), C=st_.integers(1, 17), seed=st_.integers(0, 10_000),
       t=st_.integers(1, 50), gs=st_.sampled_from([1e-4, 1e-2, 1.0]))
def test_p10_bruteforce_property(R, C, seed, t, gs):
    p, g, st = random_case(R, C, seed=seed, g_std=gs)
    flat = pack_mlp(random_mlp(seed % 7, bias_std=0.1))
    compare_one_step(p, g, st, t, flat, Hyper())
