"""Pins of the health / re-orthonormalisation oracle (CPU) against closed
forms: the polar decomposition, drift of scaled identities, statistics of
two-valued data."""

import numpy as np
import pytest

from oracle import health as H


def _orthogonal(d, seed):
    rng = np.random.default_rng(seed)
    Q, R = np.linalg.qr(rng.standard_normal((d, d)))
    return Q * np.sign(np.diag(R))


def test_drift_of_permutation_is_zero_and_of_scaled_identity_is_closed_form():
    P = np.eye(7)[[3, 0, 6, 1, 5, 2, 4]]
    assert H.orth_drift(P) == 0.0
    eps = 2.0 ** -10
    assert H.orth_drift((1 + eps) * np.eye(5)) == pytest.approx(2 * eps + eps * eps, rel=1e-12)


def test_v_stats_closed_forms():
    v = np.full((3, 4), 2.5)
    assert H.v_stats(v) == (2.5, 0.0, 2.5, 2.5)
    v = np.array([[1.0, 5.0], [1.0, 5.0]])          # two values, equal counts: std = |a - b| / 2
    m, s, lo, hi = H.v_stats(v)
    assert (m, s, lo, hi) == (3.0, 2.0, 1.0, 5.0)
    v = np.array([-2.0, 2.0])
    assert H.v_stats(v)[:2] == (2.0, 2.0)


def test_nonfinite_counts_nan_and_inf():
    a = np.zeros((4, 4)); a[0, 1] = np.nan; a[2, 2] = np.inf
    b = np.ones(5); b[4] = -np.inf
    assert H.nonfinite(a, b) == 3


@pytest.mark.parametrize("d", [1, 4, 17])
def test_polar_factor_of_orthogonal_times_spd_is_the_orthogonal_factor(d):
    Q = _orthogonal(d, d)
    rng = np.random.default_rng(100 + d)
    B = rng.standard_normal((d, d))
    S = B @ B.T + d * np.eye(d)                     # symmetric positive definite
    assert np.max(np.abs(H.polar_factor(Q @ S) - Q)) < 1e-12
    assert np.max(np.abs(H.polar_factor(Q) - Q)) < 1e-13


def test_newton_schulz_converges_quadratically_to_the_polar_factor():
    d = 12
    Q = _orthogonal(d, 3)
    rng = np.random.default_rng(4)
    E = rng.standard_normal((d, d)); E = 1e-2 * (E + E.T) / 2
    X = Q @ (np.eye(d) + E)                         # polar factor Q, drift ~ 2e-2
    errs = [np.max(np.abs(H.newton_schulz(X, k) - Q)) for k in range(5)]
    assert errs[0] > 1e-3
    for k in range(3):
        assert errs[k + 1] < 10 * errs[k] ** 2
    assert errs[4] < 1e-13


def test_planted_elementwise_square_root_reading_is_caught():
    """The printed line read literally (elementwise square root of the
    inverse Gram) does not give an orthonormal basis."""
    Q = _orthogonal(6, 9)
    X = Q @ np.diag([1.0, 1.1, 0.9, 1.2, 0.8, 1.05])
    with np.errstate(invalid="ignore"):
        literal = X @ np.sqrt(np.linalg.inv(X.T @ X))
    assert not (np.all(np.isfinite(literal)) and H.orth_drift(literal) < 1e-6)
    assert H.orth_drift(H.polar_factor(X)) < 1e-12
