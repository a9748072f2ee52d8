"""Pins of the bf16-rotation variant's oracle (CPU).

The variant is the method with its rotation matrices stored in 16-bit floats
(the pipeline-staleness page, section 3.1): U and V are rounded to bfloat16
and nothing else. Where that rounding is exact (signed-permutation or
identity bases) it must be bitwise the method; its result must depend on U,
V only through their roundings; a brute-force Kronecker evaluation of the
two-sided rotation must agree on tiny inputs; its first step is the method's;
elsewhere it must stay within the bases' rounding of the method.
"""

import numpy as np
import pytest

import oracle
from oracle import bf16_rotation as B
from tests import textbook

HP = oracle.Hyper(0.9, 0.999, 1e-8, 1e-3, 3, 1)


def signed_permutation(d, rng):
    P = np.zeros((d, d))
    P[np.arange(d), rng.permutation(d)] = rng.choice([-1.0, 1.0], d)
    return P


@pytest.mark.parametrize("shape", [(6, 9), (9, 6), (8, 8)])
def test_signed_permutation_bases_are_the_method(shape):
    """Signed permutations are orthogonal and exact in bfloat16, so rounding
    the bases changes nothing: W, v and every intermediate are bitwise the
    method's. The bases are not symmetric, so a transposed basis anywhere in
    the variant changes the result; u is not bfloat16-representable, so a
    rounding of u (not part of the method) would show."""
    m, n = shape
    rng = np.random.default_rng(3)
    U = signed_permutation(m, rng)
    V = signed_permutation(n, rng)
    assert not np.array_equal(U, U.T) and not np.array_equal(V, V.T)
    G = oracle.round_f32(rng.standard_normal((m, n)) * 1e-2)
    M = oracle.round_bf16(rng.standard_normal((m, n)) * 1e-2)
    W = oracle.round_f32(rng.standard_normal((m, n)) * 1e-2)
    v = oracle.round_f32(rng.random((m, n)) * 1e-5)
    Wm, vm, im = oracle.rotated_adam_apply(W, v, M, G, U, V, HP.beta2, HP.eps, HP.lr)
    Wb, vb, ib = B.bf16_rotation_apply(W, v, M, G, U, V, HP.beta2, HP.eps, HP.lr)
    assert np.array_equal(vb, vm) and np.array_equal(Wb, Wm)
    for k in ("Gt", "mt", "u", "dW"):
        assert np.array_equal(ib[k], im[k]), k
    assert not np.array_equal(oracle.round_bf16(im["u"]), im["u"])


def test_identity_bases_are_coordinatewise_adam():
    m, n = 5, 7
    rng = np.random.default_rng(4)
    G = textbook.f32(rng.standard_normal((m, n)) * 1e-2)
    M = oracle.round_bf16(rng.standard_normal((m, n)) * 1e-2)
    W = textbook.f32(rng.standard_normal((m, n)) * 1e-2)
    v = textbook.f32(rng.random((m, n)) * 1e-5)
    Wb, vb, _ = B.bf16_rotation_apply(W, v, M, G, np.eye(m), np.eye(n), HP.beta2, HP.eps, HP.lr)
    b2, e, a = (float(np.float32(x)) for x in (HP.beta2, HP.eps, HP.lr))
    for i in range(m):
        for j in range(n):
            vij = textbook.f32(b2 * v[i, j] + (1.0 - b2) * G[i, j] * G[i, j])
            uij = M[i, j] / (np.sqrt(vij) + e)
            assert vb[i, j] == vij
            assert Wb[i, j] == textbook.f32(W[i, j] - a * uij)


def test_result_depends_on_the_bases_only_through_their_roundings():
    """The 16-bit storage of the bases is the only rounding the variant adds:
    passing rb(U), rb(V) instead of U, V gives bitwise the same step, and
    random orthogonal bases are not bfloat16-exact, so the step differs from
    the method's."""
    m, n = 12, 20
    rng = np.random.default_rng(14)
    U, V = rand_q(m, rng), rand_q(n, rng)
    G = oracle.round_f32(rng.standard_normal((m, n)) * 1e-2)
    M = oracle.round_bf16(rng.standard_normal((m, n)) * 1e-2)
    W = oracle.round_f32(rng.standard_normal((m, n)) * 1e-2)
    v = oracle.round_f32(rng.random((m, n)) * 1e-5)
    a = B.bf16_rotation_apply(W, v, M, G, U, V, HP.beta2, HP.eps, HP.lr)
    b = B.bf16_rotation_apply(W, v, M, G, oracle.round_bf16(U), oracle.round_bf16(V), HP.beta2, HP.eps, HP.lr)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    Wm, _, _ = oracle.rotated_adam_apply(W, v, M, G, U, V, HP.beta2, HP.eps, HP.lr)
    assert not np.array_equal(a[0], Wm)


def test_two_sided_rotation_by_kronecker_brute_force():
    """vec(Ub^T X Vb) = (Vb kron Ub)^T vec(X) and vec(Ub u Vb^T) = (Vb kron
    Ub) vec(u) (column-major vec): the rotations evaluated as one Kronecker
    matrix-vector product per operand, on tiny random orthogonal bases,
    against the oracle's two-sided products."""
    m, n = 3, 5
    rng = np.random.default_rng(15)
    U, V = rand_q(m, rng), rand_q(n, rng)
    Ub, Vb = oracle.round_bf16(U), oracle.round_bf16(V)
    K = np.kron(Vb, Ub)
    vec = lambda X: X.reshape(-1, order="F")
    unvec = lambda x: x.reshape((m, n), order="F")
    G = oracle.round_f32(rng.standard_normal((m, n)) * 1e-2)
    M = oracle.round_bf16(rng.standard_normal((m, n)) * 1e-2)
    W = oracle.round_f32(rng.standard_normal((m, n)) * 1e-2)
    v = oracle.round_f32(rng.random((m, n)) * 1e-5)
    _, _, it = B.bf16_rotation_apply(W, v, M, G, U, V, HP.beta2, HP.eps, HP.lr)
    assert np.max(np.abs(unvec(K.T @ vec(G)) - it["Gt"])) <= 1e-16
    assert np.max(np.abs(unvec(K.T @ vec(M)) - it["mt"])) <= 1e-16
    assert np.max(np.abs(unvec(K @ vec(it["u"])) - it["dW"])) <= 1e-12 * np.max(np.abs(it["dW"]))


def test_planted_rounding_of_u_is_caught(monkeypatch):
    """The old reading rounded u (and the right rotations) to bfloat16 as the
    device stores them: the signed-permutation pin rejects it."""
    real = B.bf16_rotation_apply

    def rounding_u(W, v, M, G, U, V, beta2, eps, lr):
        W1, v1, it = real(W, v, M, G, U, V, beta2, eps, lr)
        ub = oracle.round_bf16(it["u"])
        dW = it["Ub"] @ ub @ it["Vb"].T
        return oracle.round_f32(W - oracle.as_f32_scalar(lr) * dW), v1, dict(it, u=ub, dW=dW)
    monkeypatch.setattr(B, "bf16_rotation_apply", rounding_u)
    with pytest.raises(AssertionError):
        test_signed_permutation_bases_are_the_method((6, 9))


def test_planted_unrounded_left_basis_is_caught(monkeypatch):
    """A variant that forgets to round U fails the roundings-only pin."""
    real_round = oracle.round_bf16
    calls = {"n": 0}

    def skip_first(x):
        calls["n"] += 1
        return np.asarray(x, np.float64) if calls["n"] % 2 == 1 else real_round(x)   # Ub unrounded
    monkeypatch.setattr(B, "round_bf16", skip_first)
    with pytest.raises(AssertionError):
        test_result_depends_on_the_bases_only_through_their_roundings()


def _trajectories(m, n, steps, seed, m_dtype="bf16"):
    rng = np.random.default_rng(seed)
    W0 = rng.standard_normal((m, n)) * 1e-2
    a = oracle.OracleState.fresh(W0, m_dtype)
    b = oracle.OracleState.fresh(W0, m_dtype)
    out = []
    for _ in range(steps):
        G = rng.standard_normal((m, n)) * 1e-2
        Wa, Wb = a.W.copy(), b.W.copy()
        oracle.step(a, G, HP)
        B.step_bf16_rotation(b, G, HP)
        out.append(((Wa - a.W), (Wb - b.W), a.last["refreshed"], b.last["bf16"]))
    return W0, a, b, out


def test_first_step_is_the_method():
    _, a, b, out = _trajectories(12, 20, 1, 5)
    dA, dB, _, bf16 = out[0]
    assert np.array_equal(dA, dB) and np.array_equal(a.v, b.v) and not bf16


@pytest.mark.parametrize("shape", [(24, 40), (40, 24), (32, 32)])
def test_apply_within_bf16_rounding_of_the_method(shape):
    """From the same established state (v from three earlier steps), the
    variant's update differs from the method's by the bfloat16 roundings of
    the bases, each entry at most 2^-9 relative, which enter the update four
    times (two in G~ through u's denominator, two in m~ and the rotation
    back): the update within 8 * 2^-9 in Frobenius norm, v within 2^-6 of its
    maximum (G~ enters squared)."""
    m, n = shape
    rng = np.random.default_rng(6)
    st = oracle.OracleState.fresh(rng.standard_normal((m, n)) * 1e-2, "bf16")
    for _ in range(3):
        oracle.step(st, rng.standard_normal((m, n)) * 1e-2, HP)
    G = oracle.round_f32(rng.standard_normal((m, n)) * 1e-2)
    M = oracle.momentum_update(st.M, G, HP.beta1, "bf16")
    _, vm, im = oracle.rotated_adam_apply(st.W, st.v, M, G, st.U, st.V, HP.beta2, HP.eps, HP.lr)
    _, vb, ib = B.bf16_rotation_apply(st.W, st.v, M, G, st.U, st.V, HP.beta2, HP.eps, HP.lr)
    rel = np.linalg.norm(ib["dW"] - im["dW"]) / np.linalg.norm(im["dW"])
    assert 1e-4 < rel <= 8 * 2.0 ** -9
    assert np.max(np.abs(vb - vm)) <= 2.0 ** -6 * np.max(vm)


def test_trajectory_stays_near_the_method_across_refreshes():
    """Seven steps with a refresh every three: the accumulated change of W
    stays within 10 % of the method's in Frobenius norm (the first bf16 step
    after the first, where v still holds one step of squares, contributes the
    most) and the gap shrinks as v accumulates."""
    W0, a, b, out = _trajectories(24, 40, 7, 7)
    cum = [np.linalg.norm(o[1] - o[0]) / np.linalg.norm(o[0]) for o in out]
    total = np.linalg.norm((b.W - W0) - (a.W - W0)) / np.linalg.norm(a.W - W0)
    assert total <= 0.1
    assert cum[-1] < cum[1]
    assert [o[2] for o in out] == [True, False, False, True, False, False, True]
    assert [o[3] for o in out] == [False] + [True] * 6


def test_first_step_in_bf16_would_be_dominated_by_roundoff():
    """Why the first step runs in binary32: with v = 0 the bf16 rotation's
    roundoff in directions where G~ is tiny is divided by eps-sized
    denominators, and the update grows well beyond the method's."""
    rng = np.random.default_rng(8)
    m, n = 24, 40
    G = oracle.round_f32(rng.standard_normal((m, n)) * 1e-2)
    M = oracle.momentum_update(np.zeros((m, n)), G, HP.beta1, "bf16")
    U, V = oracle.refresh_bases(M, np.eye(m), np.eye(n), 1)
    z = np.zeros((m, n))
    _, _, im = oracle.rotated_adam_apply(z, z, M, G, U, V, HP.beta2, HP.eps, HP.lr)
    _, _, ib = B.bf16_rotation_apply(z, z, M, G, U, V, HP.beta2, HP.eps, HP.lr)
    assert np.linalg.norm(ib["dW"]) > 1.5 * np.linalg.norm(im["dW"])


# ---- both variants together: bf16 rotations and the carried m~ -------------

@pytest.mark.parametrize("recompute", [True, False])
def test_combined_signed_permutation_bases_are_the_carried_method(recompute):
    """With signed-permutation bases the combination equals the fp32
    carried-momentum oracle bitwise: m~, v and W."""
    from oracle import rotated_momentum as RM
    m, n = 7, 10
    rng = np.random.default_rng(11)
    U, V = signed_permutation(m, rng), signed_permutation(n, rng)
    G = oracle.round_f32(rng.standard_normal((m, n)) * 1e-2)
    M = oracle.round_bf16(rng.standard_normal((m, n)) * 1e-2)
    W = oracle.round_f32(rng.standard_normal((m, n)) * 1e-2)
    v = oracle.round_f32(rng.random((m, n)) * 1e-5)
    mt0 = oracle.round_f32(rng.standard_normal((m, n)) * 1e-3)
    Wr, vr, mtr, ir = RM.rotated_momentum_apply(W, v, mt0, M, G, U, V, HP.beta1, HP.beta2, HP.eps, HP.lr, recompute)
    Wb, vb, mtb, ib = B.bf16_rotated_momentum_apply(W, v, mt0, M, G, U, V, HP.beta1, HP.beta2, HP.eps, HP.lr,
                                                    recompute)
    assert np.array_equal(mtb, mtr) and np.array_equal(vb, vr) and np.array_equal(Wb, Wr)


def test_combined_recompute_is_the_bf16_variant():
    """A recomputing step of the combination is the bf16 variant's step with
    m~ rounded to binary32 (where the device stores it)."""
    m, n = 12, 20
    rng = np.random.default_rng(12)
    U = rand_q(m, rng)
    V = rand_q(n, rng)
    G = oracle.round_f32(rng.standard_normal((m, n)) * 1e-2)
    M = oracle.round_bf16(rng.standard_normal((m, n)) * 1e-2)
    W = oracle.round_f32(rng.standard_normal((m, n)) * 1e-2)
    v = oracle.round_f32(rng.random((m, n)) * 1e-5)
    _, vb, ib = B.bf16_rotation_apply(W, v, M, G, U, V, HP.beta2, HP.eps, HP.lr)
    _, vc, mtc, ic = B.bf16_rotated_momentum_apply(W, v, None, M, G, U, V, HP.beta1, HP.beta2, HP.eps, HP.lr, True)
    assert np.array_equal(vb, vc) and np.array_equal(mtc, oracle.round_f32(ib["mt"]))


def test_combined_trajectory_stays_near_the_method():
    """Seven steps, refresh every three: within 10 % of the method's
    accumulated update; the first step is bitwise the fp32 carried-momentum
    step, then bf16 steps carry m~ between refreshes."""
    from oracle import rotated_momentum as RM
    rng = np.random.default_rng(13)
    m, n = 24, 40
    W0 = rng.standard_normal((m, n)) * 1e-2
    a = oracle.OracleState.fresh(W0, "bf16")
    b = oracle.OracleState.fresh(W0, "bf16")
    c = oracle.OracleState.fresh(W0, "bf16")
    mt, valid, recs = None, False, []
    for t in range(1, 8):
        G = rng.standard_normal((m, n)) * 1e-2
        oracle.step(a, G, HP)
        mt = B.step_bf16_rotated_momentum(b, mt, G, HP, valid)
        valid = True
        recs.append(b.last["recompute"])
        if t == 1:
            RM.step_rotated_momentum(c, None, G, HP, False)
            assert np.array_equal(c.W, b.W) and np.array_equal(c.v, b.v)
    assert recs == [True, False, False, True, False, False, True]
    assert np.linalg.norm((b.W - W0) - (a.W - W0)) / np.linalg.norm(a.W - W0) <= 0.1


def rand_q(d, rng):
    q, r = np.linalg.qr(rng.standard_normal((d, d)))
    return q * np.sign(np.diag(r))


# ---- bases stored in 16 bits -------------------------------------------------

def test_stored_bases_are_bfloat16_and_within_half_an_ulp_of_lapack():
    """After a refresh the stored bases are bfloat16 values, each within half
    a bfloat16 ulp (plus fp64 round-off) of the positive-diagonal LAPACK QR of
    the Gram matrix applied to the stored start, on the well-determined
    columns (a single pass from the identity: U = qr(M M^T))."""
    m, n = 24, 40
    rng = np.random.default_rng(21)
    M = oracle.round_bf16(rng.standard_normal((m, n)) * 1e-2)
    U16, V16 = B.refresh_bases_bf16(M, np.eye(m), np.eye(n), 1)
    assert np.array_equal(U16, oracle.round_bf16(U16)) and np.array_equal(V16, oracle.round_bf16(V16))
    q, r = np.linalg.qr(M @ M.T)
    q = q * np.where(np.diag(r) < 0, -1.0, 1.0)
    from tests.contract import ulp_bf16
    assert np.all(np.abs(U16 - q) <= 0.5 * ulp_bf16(q) + 1e-12)


def test_storage_trajectory_keeps_bases_in_16_bits_and_stays_near_the_method():
    """Seven steps with a refresh every three from 16-bit bases: the stored
    bases stay bfloat16 throughout, the refresh starts from them, and the
    accumulated update stays within 10 % of the method's after the first
    step (which, with 16-bit bases and v = 0, is large: see the module)."""
    rng = np.random.default_rng(23)
    m, n = 24, 40
    W0 = rng.standard_normal((m, n)) * 1e-2
    a = oracle.OracleState.fresh(W0, "bf16")
    b = oracle.OracleState.fresh(W0, "bf16")
    for t in range(1, 8):
        G = rng.standard_normal((m, n)) * 1e-2
        Wa, Wb = a.W.copy(), b.W.copy()
        oracle.step(a, G, HP)
        B.step_bf16_storage(b, G, HP)
        assert np.array_equal(b.U, oracle.round_bf16(b.U)) and np.array_equal(b.V, oracle.round_bf16(b.V))
        if t == 1:
            first = (np.linalg.norm(b.W - Wb), np.linalg.norm(a.W - Wa))
            W1a, W1b = a.W.copy(), b.W.copy()
    later = np.linalg.norm((b.W - W1b) - (a.W - W1a)) / np.linalg.norm(a.W - W1a)
    assert later <= 0.1
    assert first[0] > first[1]


def test_planted_binary32_storage_is_caught(monkeypatch):
    """Bases stored in binary32 instead of 16 bits fail the storage pin."""
    monkeypatch.setattr(B, "round_bf16", oracle.round_f32)
    with pytest.raises(AssertionError):
        test_stored_bases_are_bfloat16_and_within_half_an_ulp_of_lapack()
