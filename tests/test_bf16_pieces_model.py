"""CPU model of the arithmetic behind the bf16-piece products (no GPU).

The grouped GEMM's default mode and the pieced momentum product rest on two
facts, checked here in float64 with bfloat16 rounding done by torch's own
float32 -> bfloat16 cast (round to nearest even):

* an fp32 value x splits exactly into three bf16 values
  hi = rb(x), mid = rb(x - hi), lo = rb(x - hi - mid), hi + mid + lo = x;
* of the nine piece products of a b, the six kept (hi hi, hi mid, mid hi,
  hi lo, mid mid, lo hi) differ from a b by less than 2^-23 |a b|, so a dot
  product summed from them in fp32 meets the fp32 dot-product bound.

A planted mistake (dropping mid mid) must break the second bound.
"""

import numpy as np

from tests.textbook import bf16_via_torch


def split3(x):
    x = np.asarray(x, np.float32).astype(np.float64)
    hi = bf16_via_torch(x)
    r1 = (x - hi).astype(np.float32)          # exact in fp32
    mid = bf16_via_torch(r1)
    r2 = (r1.astype(np.float64) - mid).astype(np.float32)
    lo = bf16_via_torch(r2)
    return hi, mid, lo


def _samples(n, seed):
    rng = np.random.default_rng(seed)
    mag = 10.0 ** rng.uniform(-30, 30, n)
    return (rng.standard_normal(n) * mag).astype(np.float32)


def test_three_pieces_sum_exactly_to_the_fp32_value():
    x = _samples(200_000, 1)
    hi, mid, lo = split3(x)
    assert np.array_equal(hi + mid + lo, x.astype(np.float64))
    for p in (hi, mid, lo):   # every piece is a bf16 value
        assert np.array_equal(bf16_via_torch(p.astype(np.float32)), p)
    # each residual is at most half a bf16 ulp of the piece before it
    assert np.all(np.abs(mid) <= np.abs(hi) * 2.0 ** -8)
    assert np.all(np.abs(lo) <= np.abs(mid) * 2.0 ** -8)


def _six(a, b, drop_midmid=False):
    ah, am, al = split3(a)
    bh, bm, bl = split3(b)
    terms = [al * bh, am * bm, ah * bl, am * bh, ah * bm, ah * bh]
    if drop_midmid:
        terms.pop(1)
    return sum(terms)


def test_six_piece_products_are_within_one_fp32_rounding():
    a = _samples(100_000, 2)
    b = _samples(100_000, 3)
    exact = a.astype(np.float64) * b.astype(np.float64)
    six = _six(a, b)
    rel = np.abs(six - exact) / np.abs(exact)
    assert rel.max() < 2.0 ** -23, rel.max()
    planted = np.abs(_six(a, b, drop_midmid=True) - exact) / np.abs(exact)
    assert planted.max() > 2.0 ** -20


def test_six_piece_dot_products_meet_the_fp32_bound():
    """Dot products of length K, each piece product exact (as in the
    MFMA), summed in fp32 in k order: within K 2^-23 sum |a_k b_k| of the
    exact value, as an fp32 dot product is."""
    rng = np.random.default_rng(4)
    for K in (1, 16, 300, 4096):
        a = rng.standard_normal((64, K)).astype(np.float32)
        b = rng.standard_normal((64, K)).astype(np.float32)
        exact = np.sum(a.astype(np.float64) * b.astype(np.float64), axis=1)
        prods = _six(a, b)                      # float64, exact piece sums per k
        acc = np.zeros(64, np.float32)
        for k in range(K):
            acc = (acc + prods[:, k].astype(np.float32)).astype(np.float32)
        bound = K * 2.0 ** -23 * np.sum(np.abs(a.astype(np.float64) * b), axis=1)
        assert np.all(np.abs(acc - exact) <= bound), K
