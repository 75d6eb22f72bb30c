"""The arithmetic behind the bf16x8 (the default) and bf16x9 MLP paths,
checked on the host with NumPy, with the same bit operations the apply kernel
performs on each fp32 operand (the three-piece truncation split of
tests/test_bf16x6_split.py):

* each of the nine piece products is exact in fp32 (8 x 8 significant bits),
  and the nine add up to a.b exactly: bf16x9's per-product error is zero;
* bf16x8 leaves out the product of the two low pieces, below 2^-30 |a b|:
  its per-product error is at most 1/64 of one fp32 rounding (2^-24 |a b|);
* a K = 16 dot product accumulated from the 9 K exact piece products in fp32
  (smallest first, as the kernel issues them; the matrix unit's own summation
  order within an instruction is its own, and any order obeys the same
  bound) stays within the classical bound for fp32 summation of its terms,
  and its error is that of an fp32 dot product with fused multiply-adds: the
  same order of magnitude over many random dot products.
"""
import numpy as np
import pytest

from test_bf16x6_split import split3, values


def test_nine_piece_products_are_exact_and_sum_to_the_product():
    a, b = values(100_000, 12), values(100_000, 13)
    keep = (np.abs(a) > 1e-15) & (np.abs(a) < 1e15) & (np.abs(b) > 1e-15) & (np.abs(b) < 1e15)
    a, b = a[keep], b[keep]
    pa, pb = split3(a), split3(b)
    total = np.zeros(a.size)
    for i in range(3):
        for j in range(3):
            p64 = pa[i].astype(np.float64) * pb[j].astype(np.float64)
            p32 = (pa[i] * pb[j]).astype(np.float32)
            assert np.array_equal(p32.astype(np.float64), p64)       # exact in fp32
            total += p64                                               # exact in fp64 (< 53 bits wide)
    assert np.array_equal(total, a.astype(np.float64) * b.astype(np.float64))


def test_bf16x8_leaves_out_less_than_one_64th_of_a_rounding():
    a, b = values(100_000, 14), values(100_000, 15)
    keep = (np.abs(a) > 1e-15) & (np.abs(a) < 1e15) & (np.abs(b) > 1e-15) & (np.abs(b) < 1e15)
    a, b = a[keep], b[keep]
    pa, pb = split3(a), split3(b)
    total = sum(pa[i].astype(np.float64) * pb[j].astype(np.float64)
                for i in range(3) for j in range(3) if (i, j) != (2, 2))
    exact = a.astype(np.float64) * b.astype(np.float64)
    rel = np.abs(total - exact) / np.abs(exact)
    assert rel.max() < 2.0 ** -30 == 2.0 ** -24 / 64


def _dot_bf16(A, B, n_products=9):
    """fp32 accumulation of the exact piece products of every term, issued
    smallest first (ll, lm, ml, hl, lh, mm, hm, mh, hh; bf16x8 without ll),
    each product over all K before the next, as the kernel's chain of matrix
    instructions."""
    pa, pb = split3(A), split3(B)
    order = [(2, 2), (2, 1), (1, 2), (0, 2), (2, 0), (1, 1), (0, 1), (1, 0), (0, 0)][9 - n_products:]
    acc = np.zeros(A.shape[0], np.float32)
    for i, j in order:
        prod = (pa[i] * pb[j]).astype(np.float32)       # exact
        for k in range(A.shape[1]):
            acc = (acc + prod[:, k]).astype(np.float32)
    return acc


def _dot_fma(A, B):
    """fp32 dot product with fused multiply-adds (one rounding per term)."""
    acc = np.zeros(A.shape[0], np.float64)
    for k in range(A.shape[1]):
        acc = (acc + A[:, k].astype(np.float64) * B[:, k].astype(np.float64)).astype(np.float32).astype(np.float64)
    return acc


@pytest.mark.parametrize("n_products", [9, 8])
def test_dot_products_have_fp32_accuracy(n_products):
    rng = np.random.default_rng(21)
    K, N = 16, 50_000
    A = rng.standard_normal((N, K)).astype(np.float32)
    B = (rng.standard_normal((N, K)) * 10.0 ** rng.uniform(-3, 3, (N, K))).astype(np.float32)
    exact = (A.astype(np.float64) * B.astype(np.float64)).sum(axis=1)
    mag = (np.abs(A.astype(np.float64) * B.astype(np.float64))).sum(axis=1)
    x9 = _dot_bf16(A, B, n_products).astype(np.float64)
    fma = _dot_fma(A, B)
    u = 2.0 ** -24
    # classical bound for recursive summation of n_products K terms in fp32
    # (each exact; bf16x8 also leaves out below 2^-30 of each product)
    assert np.all(np.abs(x9 - exact) <= (n_products * K * u + 2.0 ** -30) * mag * (1 + 1e-6))
    e9 = np.abs(x9 - exact) / mag
    ef = np.abs(fma - exact) / mag
    # same accuracy as fp32 FMA accumulation: the mean and the tail of the
    # error relative to sum |a_k b_k| agree within a factor of 1.5
    assert np.mean(e9) <= 1.5 * np.mean(ef) and np.mean(ef) <= 1.5 * np.mean(e9)
    assert np.quantile(e9, 0.999) <= 1.5 * np.quantile(ef, 0.999)
