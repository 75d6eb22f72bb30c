"""The arithmetic behind the opt-in fp16x3 MLP path, checked on the host with
NumPy (fp16 conversions round to nearest, as v_cvt_pk_f16_f32 does):

* two pieces h = fp16(x), l = fp16(x - h) carry x to within 2^-22 |x| for
  |x| in [2^-2, 2^15] (the normal range of both pieces), and to within an
  absolute 2^-25 below it (fp16's subnormal spacing is 2^-24);
* the three products kept (hh, hl, lh) are exact in fp32 and leave out at
  most ~2^-21 |a b| in the normal range;
* the wave rescaling 2^-j of a layer-2 input m >= 2^15 (j from the exponent
  of m) always lands below 2^15, and the constant-entry shift k keeps
  bound * 2^-k below 2^15.
"""
import math

import numpy as np


def split2(x):
    x = np.asarray(x, np.float32)
    h = x.astype(np.float16).astype(np.float32)
    l = (x - h).astype(np.float32).astype(np.float16).astype(np.float32)
    return h, l


def values(n, seed, lo, hi):
    rng = np.random.default_rng(seed)
    mag = 2.0 ** rng.uniform(lo, hi, n)
    return (np.where(rng.random(n) < 0.5, -1.0, 1.0) * mag).astype(np.float32)


def test_two_pieces_carry_22_bits_in_the_normal_range():
    x = values(200_000, 1, -2, 15)
    h, l = split2(x)
    err = np.abs(x.astype(np.float64) - h.astype(np.float64) - l.astype(np.float64))
    assert np.all(err <= 2.0 ** -22 * np.abs(x.astype(np.float64)))


def test_small_values_keep_an_absolute_floor():
    x = values(200_000, 2, -30, -2)
    h, l = split2(x)
    err = np.abs(x.astype(np.float64) - h.astype(np.float64) - l.astype(np.float64))
    assert np.all(err <= 2.0 ** -25 + 2.0 ** -22 * np.abs(x.astype(np.float64)))


def test_three_products_exact_in_fp32_and_the_rest_small():
    a, b = values(100_000, 3, -2, 8), values(100_000, 4, -2, 8)
    (ah, al), (bh, bl) = split2(a), split2(b)
    total = np.zeros(a.size)
    for p, q in ((ah, bh), (ah, bl), (al, bh)):
        p64 = p.astype(np.float64) * q.astype(np.float64)
        assert np.array_equal((p * q).astype(np.float32).astype(np.float64), p64)
        total += p64
    exact = a.astype(np.float64) * b.astype(np.float64)
    assert np.max(np.abs(total - exact) / np.abs(exact)) < 2.0 ** -20.5


def test_wave_rescaling_and_constant_shift_stay_below_2_15():
    for m in np.concatenate([2.0 ** np.linspace(15, 127.9, 4000), [32768.0, 65504.0, 1e30]]):
        _, ex = math.frexp(float(m))        # m < 2^ex
        j = ex - 15 if ex > 15 else 1
        assert j >= 1 and m * 2.0 ** -j < 32768.0
    for bound in 2.0 ** np.linspace(-5, 29, 3000):
        k = 0
        while bound * 2.0 ** -k >= 32768.0:
            k += 1
        assert bound * 2.0 ** -k < 32768.0 and (k == 0 or bound * 2.0 ** -(k - 1) >= 32768.0)


def test_weight_scaling_brings_three_products_to_six_bf16_products():
    """The fp16x3 path multiplies W1 and W2 by powers of two that put each
    matrix's largest weight in [4, 8) (undone exactly through ReLU and the
    fp32 biases and last layer).  Emulated on heavy-tailed features of mean
    square 1 with the synthetic MLP weights, its split error through layers
    1-2 is then within 5 % of the six-product bf16 split's (1.11e-7 against
    1.07e-7 rms, relative), while unscaled fp16 pieces of the small weights
    (below 2^-2) lose bits: 1.77e-7."""
    import sys
    import pathlib
    sys.path.insert(0, str(pathlib.Path(__file__).resolve().parents[1]))
    from learned_optimizer_step_amd import workloads as W

    hid, nf = 32, 28
    w = W.mlp_weights().astype(np.float64)
    din = nf + 11
    W1 = w[:hid * din].reshape(hid, din)[:, :nf]
    o = hid * din + hid
    W2 = w[o:o + hid * hid].reshape(hid, hid)
    rng = np.random.default_rng(5)
    x = rng.standard_t(3, size=(nf, 20_000))
    x = (x / np.sqrt((x ** 2).mean(1, keepdims=True))).astype(np.float32).astype(np.float64)

    def f16x3(a, b):
        (ah, al), (bh, bl) = split2(a), split2(b)
        return ah.astype(np.float64) @ bl + al.astype(np.float64) @ bh + ah.astype(np.float64) @ bh

    def trunc(v):
        return (np.asarray(v, np.float32).view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32)

    def bf16x6(a, b):
        def pieces(v):
            v = np.asarray(v, np.float32)
            h = trunc(v)
            r = v - h
            m = trunc(r)
            return [t.astype(np.float64) for t in (h, m, r - m)]
        (ah, am, al), (bh, bm, bl) = pieces(a), pieces(b)
        return ah @ bl + al @ bh + am @ bm + ah @ bm + am @ bh + ah @ bh

    def pow2_to_four(m):
        return 3 - math.frexp(m)[1]

    def mlp(mm, a1, a2):
        h1 = np.maximum(mm(W1 * 2.0 ** a1, x), 0) * 2.0 ** -a1
        return np.maximum(mm(W2 * 2.0 ** a2, h1 * 2.0 ** a1), 0) * 2.0 ** -(a1 + a2), h1

    def err(mm, a1, a2):
        got, h1 = mlp(mm, a1, a2)
        exact = np.maximum(W2 @ np.maximum(W1 @ x, 0), 0)
        return float(np.sqrt(np.mean((got - exact) ** 2)) / np.sqrt(np.mean(exact ** 2)))

    a1, a2 = pow2_to_four(np.abs(W1).max()), pow2_to_four(np.abs(W2).max())
    assert a1 > 0 and a2 > 0 and 4 <= np.abs(W1).max() * 2.0 ** a1 < 8
    e6, e3, e3_plain = err(bf16x6, 0, 0), err(f16x3, a1, a2), err(f16x3, 0, 0)
    assert e3 <= e6 * 1.05 and e3_plain > 1.2 * e3, (e6, e3, e3_plain)
