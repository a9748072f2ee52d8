"""Pins of the orthogonalised-momentum (Muon-style) oracle, CPU only.

The Newton-Schulz iteration is pinned by what fixes it independently: its
limit is the orthogonal polar factor (LAPACK SVD), rank-one and orthogonal
inputs are fixed points or converge in closed form, it commutes with
orthogonal changes of basis and with transposition, it ignores positive
power-of-two scaling bitwise, and on a diagonal input it reduces to the
scalar recursion s <- 1.5 s - 0.5 s^3.
"""

import numpy as np
import pytest

import oracle
from oracle import muon


def _orth(d, seed):
    q, r = np.linalg.qr(np.random.default_rng(seed).standard_normal((d, d)))
    return q * np.sign(np.diag(r))


@pytest.mark.parametrize("shape", [(8, 8), (12, 7), (7, 12)])
def test_converges_to_the_svd_polar_factor(shape):
    m, n = shape
    p = min(m, n)
    s = np.linspace(1.0, 0.1, p)
    P = _orth(m, 1)[:, :p]
    Q = _orth(n, 2)[:, :p]
    M = (P * s) @ Q.T
    O = muon.newton_schulz_polar(M, 30)
    assert np.max(np.abs(O - muon.polar_factor_svd(M))) < 1e-12
    assert np.max(np.abs(O - P @ Q.T)) < 1e-12


def test_rank_one_input_is_a_fixed_point():
    r = np.random.default_rng(3)
    a, b = r.standard_normal(9), r.standard_normal(5)
    M = np.outer(a, b)
    expect = np.outer(a / np.linalg.norm(a), b / np.linalg.norm(b))
    for iters in (0, 1, 7):
        assert np.max(np.abs(muon.newton_schulz_polar(M, iters) - expect)) < 1e-15


def test_diagonal_input_follows_the_scalar_recursion():
    s = np.array([3.0, 1.0, 0.5, 0.25, 0.0])
    M = np.diag(s)
    x = s / np.sqrt(np.sum(s * s))
    for _ in range(4):
        x = 1.5 * x - 0.5 * x ** 3
    assert np.max(np.abs(muon.newton_schulz_polar(M, 4) - np.diag(x))) < 1e-15


def test_equivariant_and_transpose_symmetric():
    r = np.random.default_rng(4)
    M = r.standard_normal((10, 6))
    P, Q = _orth(10, 5), _orth(6, 6)
    a = muon.newton_schulz_polar(P @ M @ Q.T, 5)
    b = P @ muon.newton_schulz_polar(M, 5) @ Q.T
    assert np.max(np.abs(a - b)) < 1e-13
    assert np.max(np.abs(muon.newton_schulz_polar(M.T, 5) - muon.newton_schulz_polar(M, 5).T)) < 1e-14


def test_power_of_two_scale_is_bitwise_invariant():
    M = np.random.default_rng(7).standard_normal((6, 9))
    base = muon.newton_schulz_polar(M, 6)
    for k in (-20, -3, 5):
        assert np.array_equal(muon.newton_schulz_polar(np.ldexp(M, k), 6), base)
    assert np.array_equal(muon.newton_schulz_polar(np.zeros((3, 4)), 5), np.zeros((3, 4)))


@pytest.mark.parametrize("m_dtype", ["f32", "bf16"])
def test_apply_uses_the_method_momentum_and_a_plain_step(m_dtype):
    r = np.random.default_rng(8)
    W = oracle.round_f32(r.standard_normal((9, 14)) * 1e-2)
    M = oracle.store(r.standard_normal((9, 14)) * 1e-3, m_dtype)
    G = oracle.round_f32(r.standard_normal((9, 14)) * 1e-2)
    W1, M1, O = muon.muon_apply(W, M, G, 0.9, 1e-3, 40, m_dtype)
    assert np.array_equal(M1, oracle.momentum_update(M, G, 0.9, m_dtype))
    assert np.max(np.abs(O - muon.polar_factor_svd(M1))) < 1e-10
    assert np.array_equal(W1, oracle.round_f32(W - np.float32(1e-3) * O))
