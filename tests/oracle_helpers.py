"""Helpers shared by the oracle tests (test-side only)."""
import numpy as np

from oracle import pack_mlp, unpack_mlp, Mlp


def rng(seed):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([1234, seed])))


def random_case(R, C, seed, g_std=1e-2, warm=True):
    """fp32 p, g and a (optionally non-zero) fp32 state for an R x C tensor."""
    r = rng(seed)
    p = (r.standard_normal((R, C)) * 0.02).astype(np.float32)
    g = (r.standard_normal((R, C)) * g_std).astype(np.float32)
    if warm:
        st = {"m": (r.standard_normal((3, R, C)) * g_std).astype(np.float32),
              "v": np.abs(r.standard_normal((R, C)) * g_std ** 2).astype(np.float32),
              "r": np.abs(r.standard_normal((3, R)) * g_std ** 2).astype(np.float32),
              "c": np.abs(r.standard_normal((3, C)) * g_std ** 2).astype(np.float32)}
    else:
        st = {"m": np.zeros((3, R, C), np.float32), "v": np.zeros((R, C), np.float32),
              "r": np.zeros((3, R), np.float32), "c": np.zeros((3, C), np.float32)}
    return p, g, st


def random_mlp(seed, n_time=11, bias_std=0.1):
    r = rng(10_000 + seed)
    d_in = 28 + n_time
    m = Mlp(r.standard_normal((32, d_in)) / np.sqrt(d_in), r.standard_normal(32) * bias_std,
            r.standard_normal((32, 32)) / np.sqrt(32), r.standard_normal(32) * bias_std,
            r.standard_normal((2, 32)) / np.sqrt(32), r.standard_normal(2) * bias_std)
    return unpack_mlp(pack_mlp(m), n_time)  # round to fp32 like the packed weights


def selector_mlp(d, n_time=11):
    """MLP whose output is (dir, mag) = (x_d, 0): relu(z) - relu(-z) = z."""
    d_in = 28 + n_time
    W1 = np.zeros((32, d_in)); W1[0, d] = 1.0; W1[1, d] = -1.0
    W2 = np.zeros((32, 32)); W2[0, 0] = 1.0; W2[1, 1] = 1.0
    W3 = np.zeros((2, 32)); W3[0, 0] = 1.0; W3[0, 1] = -1.0
    return Mlp(W1, np.zeros(32), W2, np.zeros(32), W3, np.zeros(2))


def magnitude_selector_mlp(d, n_time=11):
    """(dir, mag) = (1, x_d) through the hidden layers."""
    m = selector_mlp(d, n_time)
    W3 = np.zeros((2, 32)); W3[1, 0] = 1.0; W3[1, 1] = -1.0
    return Mlp(m.W1, m.b1, m.W2, m.b2, W3, np.array([1.0, 0.0]))
