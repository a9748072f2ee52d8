"""Pins of the rotated-momentum variant's oracle (CPU): it must reduce to the
method exactly where the two coincide, and stay within rounding of it
across basis epochs."""

import numpy as np
import pytest

import oracle
from oracle import rotated_momentum as RM


def _trajectory(m, n, steps, K, m_dtype, seed, variant, power_iters=1, stale_mt=False):
    rng = np.random.default_rng(seed)
    W0 = rng.standard_normal((m, n)) * 1e-2
    hp = oracle.Hyper(0.9, 0.999, 1e-8, 1e-3, K, power_iters)
    st = oracle.OracleState.fresh(W0, m_dtype)
    mt, valid = None, False
    for t in range(1, steps + 1):
        G = rng.standard_normal((m, n)) * 1e-2
        if variant:
            if stale_mt and valid:
                # planted mistake: never recompute m~ after the first step
                b1 = oracle.as_f32_scalar(hp.beta1)
                st.t += 1
                st.M = oracle.momentum_update(st.M, oracle.round_f32(G), hp.beta1, m_dtype)
                if oracle.refresh_due(st.t, K):
                    st.U, st.V = oracle.refresh_bases(st.M, st.U, st.V, power_iters)
                st.W, st.v, mt, _ = RM.rotated_momentum_apply(st.W, st.v, mt, st.M, oracle.round_f32(G), st.U,
                                                              st.V, hp.beta1, hp.beta2, hp.eps, hp.lr, False)
            else:
                mt = RM.step_rotated_momentum(st, mt, G, hp, valid)
            valid = True
        else:
            oracle.step(st, G, hp)
    return st


def test_identity_bases_fp32_momentum_is_bitwise_the_method():
    """K = 0 (bases stay I), fp32 M: m~ = M exactly, and the carried m~
    follows the same rounded recursion as M, so both paths are bitwise equal."""
    a = _trajectory(5, 7, 6, 0, "f32", 1, variant=False)
    b = _trajectory(5, 7, 6, 0, "f32", 1, variant=True)
    assert np.array_equal(a.W, b.W) and np.array_equal(a.v, b.v)


@pytest.mark.parametrize("m_dtype", ["f32", "bf16"])
def test_across_refreshes_within_rounding_of_the_method(m_dtype):
    """Refresh every 3 steps over 8 steps: the recomputation at each refresh
    keeps the variant within storage rounding of the method."""
    a = _trajectory(9, 6, 8, 3, m_dtype, 2, variant=False)
    b = _trajectory(9, 6, 8, 3, m_dtype, 2, variant=True)
    scale = np.max(np.abs(a.W))
    tol = (1e-6 if m_dtype == "f32" else 2e-2) * scale   # bf16 M: the tolerance stated for bf16 momentum
    assert np.max(np.abs(a.W - b.W)) <= tol
    assert np.max(np.abs(a.v - b.v)) <= 1e-5 * np.max(np.abs(a.v))


def test_planted_stale_rotated_momentum_after_refresh_is_caught():
    """Carrying m~ across a basis change (no recomputation) leaves m~ in the
    old basis: the result departs from the method far beyond rounding."""
    a = _trajectory(9, 6, 8, 3, "f32", 2, variant=False)
    b = _trajectory(9, 6, 8, 3, "f32", 2, variant=True, stale_mt=True)
    assert np.max(np.abs(a.W - b.W)) > 1e-4 * np.max(np.abs(a.W))
