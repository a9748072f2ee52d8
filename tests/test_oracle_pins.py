"""Pins of the fp64 oracle against what the pages and mathematics fix.

Each pin is chosen so that a plausible mistake in the oracle (a dropped term,
a swapped operand or transpose, a wrong sign convention, a wrong completion)
fails at least one of them; the mutation tests at the end plant such mistakes
in the oracle and check that the corresponding pin catches them.
"""

import json
import math
import os

import numpy as np
import pytest

import oracle.rotated_adam as ra
from oracle import Hyper, OracleState
from tests import textbook

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rng(seed):
    return np.random.default_rng(seed)


def rand_orth(d, seed):
    q, r = np.linalg.qr(rng(seed).standard_normal((d, d)))
    return q * np.sign(np.diag(r))


# --------------------------------------------------------------------------
# storage rounding
# --------------------------------------------------------------------------

def test_bf16_rounding_matches_torch_cast():
    r = rng(0)
    x = np.concatenate([
        r.standard_normal(20000).astype(np.float32),
        (r.standard_normal(2000) * 1e-39).astype(np.float32),   # binary32 subnormals
        np.clip(r.standard_normal(2000) * 1e38, -3.3e38, 3.3e38).astype(np.float32),  # near the top
        np.array([0.0, -0.0, 1.0, -1.0], np.float32),
    ])
    # exact ties: bit patterns with the low 16 bits equal to 0x8000
    ties = (r.integers(0x00800000, 0x7f000000, 4000, dtype=np.uint32) & 0xffff0000) | 0x8000
    x = np.concatenate([x, ties.view(np.float32)])
    x = x[np.isfinite(x)]
    got = ra.round_bf16(x.astype(np.float64))
    want = textbook.bf16_via_torch(x)
    assert np.array_equal(got, want, equal_nan=True)


def test_bf16_special_values():
    x = np.array([np.nan, np.inf, -np.inf, 3.4e38, -3.4e38])
    out = ra.round_bf16(x)
    assert np.isnan(out[0]) and out[1] == np.inf and out[2] == -np.inf
    assert out[3] == np.inf and out[4] == -np.inf  # rounds past the largest bfloat16


# --------------------------------------------------------------------------
# Householder QR against LAPACK and closed forms
# --------------------------------------------------------------------------

@pytest.mark.parametrize("d", [1, 2, 3, 7, 37, 64, 130])
def test_orthonormal_factor_matches_lapack(d):
    Z = rng(d).standard_normal((d, d))
    Q = ra.orthonormal_factor(Z)
    q, r = np.linalg.qr(Z)                       # LAPACK dgeqrf + dorgqr
    q = q * np.where(np.diag(r) < 0, -1.0, 1.0)
    assert np.max(np.abs(Q - q)) < 1e-12 * d
    R = Q.T @ Z
    assert np.max(np.abs(np.tril(R, -1))) < 1e-12 * d * np.max(np.abs(Z))
    assert np.all(np.diag(R) > 0)


def test_householder_qr_reconstructs_and_is_orthogonal():
    Z = rng(5).standard_normal((50, 50)) * np.logspace(0, -6, 50)[None, :]
    Q, R = ra.householder_qr(Z)
    assert np.max(np.abs(Q @ R - Z)) < 1e-13
    assert np.max(np.abs(Q.T @ Q - np.eye(50))) < 1e-13
    assert np.array_equal(R, np.triu(R))


def test_orthonormal_factor_zero_matrix_is_identity():
    # every reflector is the identity and every diagonal of R is 0 -> sign +
    assert np.array_equal(ra.orthonormal_factor(np.zeros((6, 6))), np.eye(6))


def test_orthonormal_factor_diagonal_signs():
    D = np.diag([3.0, -2.0, 0.5, -1e-3])
    Q = ra.orthonormal_factor(D)
    assert np.allclose(Q, np.diag([1.0, -1.0, 1.0, -1.0]), atol=0)


@pytest.mark.parametrize("rows,cols,k", [(40, 40, 7), (300, 64, 64), (300, 64, 1), (128, 96, 50)])
def test_thin_orthonormal_factor_matches_lapack_reduced_qr(rows, cols, k):
    """The leading k columns of the positive-diagonal Q, formed without the
    rest, against LAPACK's reduced QR (dgeqrf + dorgqr) with the same signs,
    and against the leading columns of the full factor."""
    Z = rng(rows + k).standard_normal((rows, cols)) * np.logspace(0, -3, cols)[None, :]
    Qk = ra.orthonormal_factor(Z, q_cols=k)
    assert Qk.shape == (rows, k)
    q, r = np.linalg.qr(Z[:, :k], mode="reduced")
    q = q * np.where(np.diag(r) < 0, -1.0, 1.0)
    assert np.max(np.abs(Qk - q)) < 1e-11
    if rows == cols:
        assert np.max(np.abs(Qk - ra.orthonormal_factor(Z)[:, :k])) < 1e-13


@pytest.mark.parametrize("shape,p,side", [((60, 24), 1, "U"), ((60, 24), 2, "V"), ((24, 60), 3, "U"),
                                          ((33, 33), 2, "V")])
def test_leading_subspace_iteration_equals_the_full_iteration(shape, p, side):
    """The leading k <= r columns of the refresh, iterated on their own,
    equal those of the full orthogonal iteration with completion, from a
    random orthogonal start."""
    m, n = shape
    M = rng(m * n + p).standard_normal(shape) * np.logspace(0, -1, n)[None, :]
    d = m if side == "U" else n
    X0 = rand_orth(d, 3 + p)
    A = M @ M.T if side == "U" else M.T @ M
    full = ra.subspace_iteration(A, X0, min(m, n), p)
    k = min(m, n) - 3
    lead = ra.leading_subspace_iteration(M, X0[:, :k], side, p)
    assert np.max(np.abs(lead - full[:, :k])) < 1e-11


def test_planted_transposed_gram_in_the_leading_iteration_is_caught(monkeypatch):
    """The leading-column iteration on the wrong Gram matrix (V's operator
    for U) fails the comparison with the full iteration."""
    M = rng(9).standard_normal((30, 30)) * np.logspace(0, -1, 30)[None, :]
    X0 = rand_orth(30, 4)
    full = ra.subspace_iteration(M @ M.T, X0, 30, 1)
    wrong = ra.leading_subspace_iteration(M, X0[:, :10], "V", 1)
    assert np.max(np.abs(wrong - full[:, :10])) > 1e-3


# --------------------------------------------------------------------------
# Refresh: orthogonal iteration
# --------------------------------------------------------------------------

@pytest.mark.parametrize("shape,p", [((8, 8), 1), ((16, 40), 2), ((40, 16), 1), ((33, 17), 3)])
def test_refresh_orthonormal(shape, p):
    m, n = shape
    M = rng(m * n).standard_normal(shape)
    r = min(m, n)
    U = ra.subspace_iteration(M @ M.T, np.eye(m), r, p)
    V = ra.subspace_iteration(M.T @ M, np.eye(n), r, p)
    assert np.max(np.abs(U.T @ U - np.eye(m))) <= 1e-10
    assert np.max(np.abs(V.T @ V - np.eye(n))) <= 1e-10
    Uf, Vf = ra.refresh_bases(M, np.eye(m), np.eye(n), p)
    assert np.max(np.abs(Uf - U)) < 1e-6 and np.max(np.abs(Vf - V)) < 1e-6
    assert np.array_equal(Uf, ra.round_f32(Uf))


def test_power_iteration_converges_to_eigenvectors():
    """8x8 M with singular values 2^-i: 60 passes reach the eigenbasis of M M^T."""
    P, Q = rand_orth(8, 1), rand_orth(8, 2)
    M = P @ np.diag(2.0 ** -np.arange(8)) @ Q.T
    U = ra.subspace_iteration(M @ M.T, np.eye(8), 8, 60)
    V = ra.subspace_iteration(M.T @ M, np.eye(8), 8, 60)
    for X, A in ((U, M @ M.T), (V, M.T @ M)):
        w, E = np.linalg.eigh(A)
        E = E[:, np.argsort(w)[::-1]]
        C = X.T @ E
        assert np.max(np.abs(np.abs(np.diag(C)) - 1.0)) < 1e-12
        assert np.max(np.abs(C - np.diag(np.diag(C)))) < 1e-10


def test_one_refresh_square_equals_lapack_qr_of_gram():
    M = rng(11).standard_normal((12, 12))
    U, V = ra.refresh_bases(M, np.eye(12), np.eye(12), 1)
    for X, A in ((U, M @ M.T), (V, M.T @ M)):
        q, r = np.linalg.qr(A)
        q = q * np.where(np.diag(r) < 0, -1.0, 1.0)
        # columns the Gram's conditioning leaves well determined
        assert np.max(np.abs(X[:, :4] - q[:, :4])) < 1e-6


def test_rank_one_gradient_closed_form():
    a = rng(3).standard_normal(6)
    b = rng(4).standard_normal(9)
    a[0], b[0] = -abs(a[0]) - 0.1, abs(b[0]) + 0.1
    st = OracleState.fresh(np.zeros((6, 9)))
    hp = Hyper(K=1, power_iters=1)
    ra.step(st, np.outer(a, b), hp)
    u0 = np.sign(a[0]) * a / np.linalg.norm(a)
    v0 = np.sign(b[0]) * b / np.linalg.norm(b)
    assert np.max(np.abs(st.U[:, 0] - u0)) < 1e-6   # bases stored as binary32
    assert np.max(np.abs(st.V[:, 0] - v0)) < 1e-6


def test_completion_is_qr_of_projected_previous_basis():
    m, n = 5, 11
    M = rng(21).standard_normal((m, n))
    V0 = rand_orth(n, 22)
    V = ra.subspace_iteration(M.T @ M, V0, m, 1)
    Vr = V[:, :m]
    P = (np.eye(n) - Vr @ Vr.T) @ V0[:, m:]
    q, r = np.linalg.qr(P)
    q = q * np.where(np.diag(r) < 0, -1.0, 1.0)
    assert np.max(np.abs(V[:, m:] - q)) < 1e-10
    # and the leading block spans the range of M^T M V0[:, :m]
    Y = (M.T @ M) @ V0[:, :m]
    q1, r1 = np.linalg.qr(Y)
    assert np.max(np.abs(np.abs(Vr.T @ q1) - np.eye(m))) < 1e-10


def test_equivariance_under_orthogonal_change_of_basis():
    m, n = 7, 10
    M = rng(31).standard_normal((m, n))
    G = rng(32).standard_normal((m, n))
    W = rng(33).standard_normal((m, n))
    v = rng(34).random((m, n))
    P, Q = rand_orth(m, 35), rand_orth(n, 36)
    U0, V0 = rand_orth(m, 37), rand_orth(n, 38)
    U1 = ra.subspace_iteration(M @ M.T, U0, min(m, n), 2)
    V1 = ra.subspace_iteration(M.T @ M, V0, min(m, n), 2)
    M2 = P @ M @ Q.T
    U2 = ra.subspace_iteration(M2 @ M2.T, P @ U0, min(m, n), 2)
    V2 = ra.subspace_iteration(M2.T @ M2, Q @ V0, min(m, n), 2)
    assert np.max(np.abs(U2 - P @ U1)) < 1e-10
    assert np.max(np.abs(V2 - Q @ V1)) < 1e-10
    _, _, i1 = ra.rotated_adam_apply(W, v, M, G, U1, V1, 0.999, 1e-8, 1e-3)
    _, _, i2 = ra.rotated_adam_apply(P @ W @ Q.T, v, M2, P @ G @ Q.T, P @ U1, Q @ V1,
                                     0.999, 1e-8, 1e-3)
    assert np.max(np.abs(i2["dW"] - P @ i1["dW"] @ Q.T)) < 1e-10 * np.max(np.abs(i1["dW"]))


def test_rotation_round_trip():
    m, n = 9, 14
    M = rng(41).standard_normal((m, n))
    G = rng(42).standard_normal((m, n))
    U = ra.subspace_iteration(M @ M.T, np.eye(m), m, 1)
    V = ra.subspace_iteration(M.T @ M, np.eye(n), m, 1)
    _, _, it = ra.rotated_adam_apply(np.zeros((m, n)), np.ones((m, n)), M, G, U, V,
                                     0.999, 1e-8, 1e-3)
    scale = np.max(np.abs(G))
    assert np.max(np.abs(U @ it["Gt"] @ V.T - G)) < 1e-12 * scale
    assert np.max(np.abs(U @ it["mt"] @ V.T - M)) < 1e-12 * np.max(np.abs(M))
    assert np.max(np.abs(U.T @ it["dW"] @ V - it["u"])) < 1e-12 * np.max(np.abs(it["u"]))


# --------------------------------------------------------------------------
# Whole step: special cases and closed forms
# --------------------------------------------------------------------------

@pytest.mark.parametrize("m_dtype", ["f32", "bf16"])
def test_identity_bases_reduce_to_coordinatewise_adam(m_dtype):
    """With U = I, V = I and no refresh the step is coordinate-wise Adam, bitwise.

    The bfloat16 storage rounding is the oracle's own (pinned against torch's
    cast above); everything else on the textbook side is element by element.
    """
    m, n = 6, 5
    hp = Hyper(beta1=0.9, beta2=0.999, eps=1e-8, lr=1e-3, K=0)
    W0 = ra.round_f32(rng(51).standard_normal((m, n)) * 1e-2)
    st = OracleState.fresh(W0, m_dtype)
    w, mm, vv = W0.copy(), np.zeros((m, n)), np.zeros((m, n))
    rnd = textbook.f32 if m_dtype == "f32" else ra.round_bf16
    for t in range(4):
        G = ra.round_f32(rng(60 + t).standard_normal((m, n)) * 1e-2)
        ra.step(st, G, hp)
        w, mm, vv = textbook.adam_coordinatewise(w, mm, vv, G, 0.9, 0.999, 1e-8, 1e-3, rnd)
        assert np.array_equal(st.M, mm) and np.array_equal(st.v, vv) and np.array_equal(st.W, w)


def test_constant_gradient_fixed_basis_closed_form():
    m, n, T = 5, 8, 6
    hp = Hyper(K=0)
    b1, b2, eps, lr = (float(np.float32(x)) for x in (hp.beta1, hp.beta2, hp.eps, hp.lr))
    U, V = rand_orth(m, 71), rand_orth(n, 72)
    G = ra.round_f32(rng(73).standard_normal((m, n)) * 1e-2)
    st = OracleState.fresh(np.zeros((m, n)))
    st.U, st.V = U, V
    Gt = U.T @ G @ V
    dW = np.zeros((m, n))
    for t in range(1, T + 1):
        ra.step(st, G, hp)
        Mt = (1 - b1 ** t) * G
        vt = (1 - b2 ** t) * Gt * Gt
        ut = (1 - b1 ** t) * Gt / (np.sqrt(1 - b2 ** t) * np.abs(Gt) + eps)
        dW += U @ ut @ V.T
        assert np.max(np.abs(st.M - Mt)) < 1e-6 * np.max(np.abs(Mt))
        assert np.max(np.abs(st.v - vt)) < 1e-6 * np.max(vt)
        assert np.max(np.abs(st.W + lr * dW)) < 1e-5 * lr * np.max(np.abs(dW))


@pytest.mark.parametrize("m_dtype", ["f32", "bf16"])
def test_power_of_two_scale_invariance(m_dtype):
    """Scaling G by 2^k scales M, G~, m~ by 2^k and v by 4^k exactly; with eps = 0
    the bases and the whole weight trajectory are bitwise unchanged."""
    m, n = 6, 9
    hp = Hyper(eps=0.0, K=2, power_iters=2)
    W0 = ra.round_f32(rng(81).standard_normal((m, n)) * 1e-2)
    a, b = OracleState.fresh(W0, m_dtype), OracleState.fresh(W0, m_dtype)
    for t in range(5):
        G = ra.round_f32(rng(90 + t).standard_normal((m, n)) * 1e-2)
        ra.step(a, G, hp)
        ra.step(b, G * 2.0 ** 7, hp)
        assert np.array_equal(a.U, b.U) and np.array_equal(a.V, b.V)
        assert np.array_equal(a.W, b.W)
        assert np.array_equal(a.v * 4.0 ** 7, b.v)


def test_refresh_cadence():
    assert [t for t in range(1, 25) if ra.refresh_due(t, 10)] == [1, 11, 21]
    assert [t for t in range(1, 6) if ra.refresh_due(t, 1)] == [1, 2, 3, 4, 5]
    assert not any(ra.refresh_due(t, 0) for t in range(1, 50))


def test_refresh_keeps_t_and_uses_new_momentum():
    """The refresh in a due step sees the momentum already updated with this G."""
    m, n = 4, 6
    hp = Hyper(K=1, power_iters=3)
    G = ra.round_f32(rng(101).standard_normal((m, n)))
    st = OracleState.fresh(np.zeros((m, n)))
    ra.step(st, G, hp)
    U, V = ra.refresh_bases(ra.momentum_update(np.zeros((m, n)), G, hp.beta1, "f32"),
                            np.eye(m), np.eye(n), 3)
    assert np.array_equal(st.U, U) and np.array_equal(st.V, V)
    assert st.t == 1


# --------------------------------------------------------------------------
# arithmetic of the oracle in 50-digit arithmetic
# --------------------------------------------------------------------------

def _mp_qr_pos(Z):
    """Modified Gram-Schmidt in mpmath: the positive-diagonal Q of full-rank Z."""
    import mpmath as mp
    d = Z.rows
    Q = Z.copy()
    for j in range(d):
        for i in range(j):
            c = sum(Q[k, i] * Q[k, j] for k in range(d))
            for k in range(d):
                Q[k, j] -= c * Q[k, i]
        nrm = mp.sqrt(sum(Q[k, j] ** 2 for k in range(d)))
        for k in range(d):
            Q[k, j] /= nrm
    return Q


@pytest.mark.parametrize("shape", [(3, 5), (5, 3)])
def test_oracle_arithmetic_against_mpmath(shape):
    import mpmath as mp
    mp.mp.dps = 50
    m, n = shape
    r = min(m, n)
    M = rng(111).standard_normal(shape)
    G = rng(112).standard_normal(shape)
    v = rng(113).random(shape)
    U = ra.subspace_iteration(M @ M.T, np.eye(m), r, 2)
    V = ra.subspace_iteration(M.T @ M, np.eye(n), r, 2)
    _, _, it = ra.rotated_adam_apply(np.zeros(shape), v, M, G, U, V, 0.999, 1e-8, 1e-3)

    Mm = mp.matrix(M.tolist())
    def iterate(A, d):
        X = mp.eye(d)
        for _ in range(2):
            Y = A * X
            Z = mp.matrix(d, d)
            for i in range(d):
                for j in range(d):
                    Z[i, j] = Y[i, j] if j < r else X[i, j]
            X = _mp_qr_pos(Z)
        return X
    Um = iterate(Mm * Mm.T, m)
    Vm = iterate(Mm.T * Mm, n)
    to_np = lambda A: np.array([[float(A[i, j]) for j in range(A.cols)] for i in range(A.rows)])
    assert np.max(np.abs(to_np(Um) - U)) < 1e-13
    assert np.max(np.abs(to_np(Vm) - V)) < 1e-13
    Gt = Um.T * mp.matrix(G.tolist()) * Vm
    assert np.max(np.abs(to_np(Gt) - it["Gt"])) < 1e-13 * np.max(np.abs(it["Gt"]))


# --------------------------------------------------------------------------
# stored regression fixture (written by tests/golden/make_golden.py)
# --------------------------------------------------------------------------

def test_golden_tiny_trajectory():
    from tests.golden.make_golden import tiny_trajectory
    with open(os.path.join(GOLDEN, "tiny_trajectory.json")) as f:
        want = json.load(f)
    got = tiny_trajectory()
    assert got.keys() == want.keys()
    for k in want:
        assert np.allclose(got[k], want[k], rtol=1e-12, atol=0), k


# --------------------------------------------------------------------------
# planted mistakes: each must be caught by the pin that targets it
# --------------------------------------------------------------------------

def _fails(fn):
    try:
        fn()
    except AssertionError:
        return True
    return False


def test_planted_missing_sign_fix_is_caught(monkeypatch):
    monkeypatch.setattr(ra, "orthonormal_factor", lambda Z: ra.householder_qr(Z)[0])
    assert _fails(lambda: test_orthonormal_factor_matches_lapack(37))


def test_planted_transposed_right_basis_is_caught(monkeypatch):
    orig = ra.rotated_adam_apply

    def bad(W, v, M, G, U, V, *a):
        return orig(W, v, M, G, U, np.asarray(V).T, *a)
    monkeypatch.setattr(ra, "rotated_adam_apply", bad)
    assert _fails(test_constant_gradient_fixed_basis_closed_form)


def test_planted_wrong_completion_is_caught(monkeypatch):
    def bad(A, X, rank, passes):
        for _ in range(passes):
            X = ra.orthonormal_factor(A @ X + 1e-3 * X)
        return X
    monkeypatch.setattr(ra, "subspace_iteration", bad)
    assert _fails(test_completion_is_qr_of_projected_previous_basis)


def test_planted_unsquared_second_moment_is_caught(monkeypatch):
    monkeypatch.setattr(ra, "rotated_adam_apply", _adam_without_square)
    assert _fails(lambda: test_power_of_two_scale_invariance("f32"))


def _adam_without_square(W, v, M, G, U, V, beta2, eps, lr):
    Gt = U.T @ G @ V
    mt = U.T @ M @ V
    v_new = ra.round_f32(beta2 * v + (1 - beta2) * np.abs(Gt))
    u = mt / (np.sqrt(v_new) + eps)
    dW = U @ u @ V.T
    return ra.round_f32(W - lr * dW), v_new, {"Gt": Gt, "mt": mt, "u": u, "dW": dW}


def test_planted_bias_correction_is_caught(monkeypatch):
    orig = ra.rotated_adam_apply

    def bad(W, v, M, G, U, V, beta2, eps, lr):
        return orig(W, v, M / 0.1, G, U, V, beta2, eps, lr)
    monkeypatch.setattr(ra, "rotated_adam_apply", bad)
    assert _fails(lambda: test_identity_bases_reduce_to_coordinatewise_adam("f32"))
