"""The arithmetic behind the bf16x6 MLP path, checked on the host with NumPy
(the same bit operations the apply kernel performs on each fp32 operand):

* x = h + m + l exactly, where h is x with its low 16 bits cleared, m the same
  of r = x - h (exact in fp32), and l = r - m, which is itself a bf16 value;
  |m| < 2^-7 |x| and |l| < 2^-15 |x|;
* the six piece products the kernel keeps (hh, hm, mh, hl, lh, mm) are exact
  in fp32, and the three it leaves out stay below 2^-21 |a b|, with a median
  below one fp32 rounding (2^-24).
"""
import numpy as np

MASK = np.uint32(0xFFFF0000)


def split3(x):
    x = np.asarray(x, np.float32)
    h = (x.view(np.uint32) & MASK).view(np.float32)
    r = (x - h).astype(np.float32)
    m = (r.view(np.uint32) & MASK).view(np.float32)
    l = (r - m).astype(np.float32)
    return h, m, l


def values(n, seed):
    rng = np.random.default_rng(seed)
    mag = 10.0 ** rng.uniform(-20, 20, n)
    return (np.where(rng.random(n) < 0.5, -1.0, 1.0) * mag * rng.uniform(1, 2, n)).astype(np.float32)


def test_three_pieces_rebuild_x_exactly_and_are_bf16():
    x = np.concatenate([values(200_000, 1), np.float32([0.0, -0.0, 1.0, -1.0, 3.0, 1 / 3, np.pi, 65504.0])])
    h, m, l = split3(x)
    for piece in (h, m, l):
        assert not np.any(piece.view(np.uint32) & np.uint32(0xFFFF))
    assert np.array_equal(h.astype(np.float64) + m.astype(np.float64) + l.astype(np.float64), x.astype(np.float64))
    nz = x != 0
    ax = np.abs(x[nz]).astype(np.float64)
    assert np.all(np.abs(m[nz]) < 2.0 ** -7 * ax)
    assert np.all(np.abs(l[nz]) < 2.0 ** -15 * ax)


def test_six_piece_products_are_exact_in_fp32_and_the_rest_is_small():
    a, b = values(100_000, 2), values(100_000, 3)
    pa, pb = split3(a), split3(b)
    kept = [(0, 0), (0, 1), (1, 0), (0, 2), (2, 0), (1, 1)]
    total = np.zeros(a.size)
    for i, j in kept:
        p64 = pa[i].astype(np.float64) * pb[j].astype(np.float64)
        with np.errstate(over="ignore"):
            p32 = (pa[i] * pb[j]).astype(np.float32)
        fin = np.isfinite(p32) & (np.abs(p64) > 1e-37)  # normal fp32 range
        assert np.array_equal(p32[fin].astype(np.float64), p64[fin])
        total += p64
    exact = a.astype(np.float64) * b.astype(np.float64)
    ok = np.abs(exact) > 1e-30
    rel = np.abs(total[ok] - exact[ok]) / np.abs(exact[ok])
    assert rel.max() < 2.0 ** -21
    assert np.median(rel) < 2.0 ** -24
