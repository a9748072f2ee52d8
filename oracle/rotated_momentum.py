"""Plain fp64 CPU oracle of the rotated-momentum variant of the step.

TEST INFRASTRUCTURE. Only ``tests/`` and ``__graft_entry__.smoke()`` may
import or call this module; it shares no code with the HIP path.

The method ([P3] "Pipeline parallelism and gradient staleness optimisation in
distributed training", section 2.2) rotates the momentum matrix into the
current basis every step, m~ = U^T M V. Within one basis epoch (the steps
between two refreshes) U and V do not change and the momentum is an EMA
([P2] section 2.2), so by linearity

    U^T M_t V = b1 U^T M_{t-1} V + (1 - b1) U^T G_t V = b1 m~_{t-1} + (1 - b1) G~_t,

and m~ can be carried in rotated coordinates: each step then needs the
rotation of G and the rotation back only, two two-sided products instead of
three. M itself is still kept in the original space, because a refresh
builds the new bases from it; at a refresh (and whenever m~ is not known for
the current bases) m~ is recomputed as U^T M V. The variant agrees with the
method in exact arithmetic and differs only in rounding (m~ is stored in
binary32 instead of being recomputed from the stored M).
"""

from __future__ import annotations

import numpy as np

from .rotated_adam import (Hyper, OracleState, as_f32_scalar, momentum_update, refresh_bases,
                           refresh_due, round_f32)

__all__ = ["rotated_momentum_apply", "step_rotated_momentum"]


def rotated_momentum_apply(W, v, mt_prev, M, G, U, V, beta1: float, beta2: float, eps: float, lr: float,
                           recompute: bool):
    """One step in rotated coordinates with a carried m~.

    recompute: m~ = U^T M V (M the stored momentum, already updated this
    step); otherwise m~ = b1 m~_prev + (1 - b1) U^T G V. m~ and v are stored
    as binary32 and u uses the stored values; W <- W - lr U u V^T.
    Returns (W_new, v_new, mt_new, intermediates)."""
    b1 = as_f32_scalar(beta1)
    b2 = as_f32_scalar(beta2)
    eps = as_f32_scalar(eps)
    lr = as_f32_scalar(lr)
    U = np.asarray(U, np.float64)
    V = np.asarray(V, np.float64)
    Gt = U.T @ np.asarray(G, np.float64) @ V
    if recompute:
        mt = round_f32(U.T @ np.asarray(M, np.float64) @ V)
    else:
        mt = round_f32(b1 * np.asarray(mt_prev, np.float64) + (1.0 - b1) * Gt)
    v_new = round_f32(b2 * np.asarray(v, np.float64) + (1.0 - b2) * (Gt * Gt))
    u = mt / (np.sqrt(v_new) + eps)
    dW = U @ u @ V.T
    W_new = round_f32(np.asarray(W, np.float64) - lr * dW)
    return W_new, v_new, mt, {"Gt": Gt, "mt": mt, "u": u, "dW": dW}


def step_rotated_momentum(state: OracleState, mt, G, hp: Hyper, mt_valid: bool):
    """One step of the variant on one matrix (momentum -> refresh -> rotate ->
    moments -> apply, as the method). ``mt`` is the carried m~ (ignored when
    ``mt_valid`` is false: the first step, or after the bases changed outside
    a step). Returns the new m~; ``state`` is updated in place."""
    G = round_f32(G)
    state.t += 1
    state.M = momentum_update(state.M, G, hp.beta1, state.m_dtype)
    refreshed = refresh_due(state.t, hp.K)
    if refreshed:
        state.U, state.V = refresh_bases(state.M, state.U, state.V, hp.power_iters)
    state.W, state.v, mt_new, inter = rotated_momentum_apply(
        state.W, state.v, mt, state.M, G, state.U, state.V, hp.beta1, hp.beta2, hp.eps, hp.lr,
        recompute=refreshed or not mt_valid)
    state.last = dict(inter, refreshed=refreshed)
    return mt_new
