"""Plain fp64 CPU oracle of the bf16-rotation variant of the step.

TEST INFRASTRUCTURE. Only ``tests/`` and ``__graft_entry__.smoke()`` may
import or call this module; it shares no code with the HIP path.

[P3] "Pipeline parallelism and gradient staleness optimisation in distributed
training", section 3.1 (mixed-precision configuration), keeps the rotation
matrices in a 16-bit float format, on the grounds that the rotation is
insensitive to their rounding. That is all this oracle rounds beyond the
method: the step rotates with the 16-bit bases Ub = rb(U), Vb = rb(V) (rb =
round to bfloat16, ties to even; bfloat16 rather than the page's float16 is a
reading: it keeps the binary32 exponent range and is the momentum's format in
[P2] "Large-model distributed optimisation: three-layer decoupling of
communication, memory and compute", section 3.3), and every product is exact:

    Ub = rb(U), Vb = rb(V)
    G~ = Ub^T G Vb,  m~ = Ub^T M Vb              (M as stored: bf16 or binary32)
    v  <- rf(b2 v + (1 - b2) G~^2);  u = m~ / (sqrt(v) + eps)
    W  <- rf(W - lr Ub u Vb^T)

The device computes these products on bf16 operands with binary32
accumulation, so it also rounds G (and an fp32 M), the right rotations G Vb
and M Vb, u and u Vb^T to bfloat16. Those roundings are an implementation's,
not the method's: the parity gate bounds them as errors (tests/contract.py,
gate_apply_bf16) instead of this oracle reproducing them.

The first step (t = 1) runs the method's own binary32 rotations. There v is
zero, so u = m~ / (sqrt(v) + eps) turns every entry of G~ that is zero in
exact arithmetic (after the step-1 refresh from M = (1 - b1) G, all of G~ off
its leading diagonal) into (1 - b1) / sqrt(1 - b2) times the sign of its
rounding error whenever that error exceeds eps / sqrt(1 - b2); a rotation
with 16-bit bases has errors of that size (2^-9 relative against 3e-7 for the
default eps), which would make the first update a full-size step in
roundoff directions. From t = 2 on v holds the first step's squares and the
rounding enters only at its own relative size.
"""

from __future__ import annotations

import numpy as np

from .rotated_adam import (Hyper, OracleState, as_f32_scalar, momentum_update, refresh_bases,
                           refresh_due, rotated_adam_apply, round_bf16, round_f32, subspace_iteration)

__all__ = ["bf16_rotation_apply", "step_bf16_rotation", "bf16_rotated_momentum_apply",
           "step_bf16_rotated_momentum", "refresh_bases_bf16", "step_bf16_storage"]


def bf16_rotation_apply(W, v, M, G, U, V, beta2: float, eps: float, lr: float):
    """Rotate, run the Adam moments and apply with the bases rounded to
    bfloat16, every product exact (the module docstring's formulas).

    Returns (W_new, v_new, intermediates) with the float64 values of Ub, Vb,
    SG = G Vb, SM = M Vb, Gt, mt, u, P = u Vb^T and dW = Ub P."""
    b2 = as_f32_scalar(beta2)
    eps = as_f32_scalar(eps)
    lr = as_f32_scalar(lr)
    Ub = round_bf16(U)
    Vb = round_bf16(V)
    SG = np.asarray(G, np.float64) @ Vb
    SM = np.asarray(M, np.float64) @ Vb
    Gt = Ub.T @ SG
    mt = Ub.T @ SM
    v_new = round_f32(b2 * np.asarray(v, np.float64) + (1.0 - b2) * (Gt * Gt))
    u = mt / (np.sqrt(v_new) + eps)
    P = u @ Vb.T
    dW = Ub @ P
    W_new = round_f32(np.asarray(W, np.float64) - lr * dW)
    return W_new, v_new, {"Ub": Ub, "Vb": Vb, "SG": SG, "SM": SM, "Gt": Gt, "mt": mt, "u": u,
                          "P": P, "dW": dW}


def step_bf16_rotation(state: OracleState, G, hp: Hyper) -> OracleState:
    """One step of the variant on one matrix: momentum and refresh as the
    method (binary32 bases), then bf16_rotation_apply, except at t = 1, where
    the method's rotated_adam_apply runs. Mutates and returns ``state``."""
    G = round_f32(G)
    state.t += 1
    state.M = momentum_update(state.M, G, hp.beta1, state.m_dtype)
    refreshed = refresh_due(state.t, hp.K)
    if refreshed:
        state.U, state.V = refresh_bases(state.M, state.U, state.V, hp.power_iters)
    apply = rotated_adam_apply if state.t == 1 else bf16_rotation_apply
    state.W, state.v, inter = apply(state.W, state.v, state.M, G, state.U, state.V, hp.beta2, hp.eps, hp.lr)
    state.last = dict(inter, refreshed=refreshed, bf16=state.t != 1)
    return state


def bf16_rotated_momentum_apply(W, v, mt_prev, M, G, U, V, beta1: float, beta2: float, eps: float, lr: float,
                                recompute: bool):
    """Both variants together: the bases rounded to bfloat16 as in
    bf16_rotation_apply, and m~ carried in binary32 within a basis epoch as
    in oracle/rotated_momentum.py. recompute: m~ = rf(Ub^T M Vb); otherwise
    m~ = rf(b1 m~_prev + (1 - b1) G~), with G~ = Ub^T G Vb. Every product
    exact. Returns (W_new, v_new, mt_new, intermediates)."""
    b1 = as_f32_scalar(beta1)
    b2 = as_f32_scalar(beta2)
    eps = as_f32_scalar(eps)
    lr = as_f32_scalar(lr)
    Ub = round_bf16(U)
    Vb = round_bf16(V)
    SG = np.asarray(G, np.float64) @ Vb
    Gt = Ub.T @ SG
    if recompute:
        SM = np.asarray(M, np.float64) @ Vb
        mt = round_f32(Ub.T @ SM)
    else:
        SM = None
        mt = round_f32(b1 * np.asarray(mt_prev, np.float64) + (1.0 - b1) * Gt)
    v_new = round_f32(b2 * np.asarray(v, np.float64) + (1.0 - b2) * (Gt * Gt))
    u = mt / (np.sqrt(v_new) + eps)
    P = u @ Vb.T
    dW = Ub @ P
    W_new = round_f32(np.asarray(W, np.float64) - lr * dW)
    return W_new, v_new, mt, {"Ub": Ub, "Vb": Vb, "SG": SG, "SM": SM, "Gt": Gt, "mt": mt, "u": u,
                              "P": P, "dW": dW}


def step_bf16_rotated_momentum(state: OracleState, mt, G, hp: Hyper, mt_valid: bool):
    """One step of the two variants together on one matrix. The first step
    (t = 1) is the fp32 rotated-momentum step (recomputing m~); later steps
    use bf16_rotated_momentum_apply, recomputing m~ at refreshes and whenever
    it is not valid. Returns the new m~; ``state`` is updated in place."""
    from .rotated_momentum import rotated_momentum_apply
    G = round_f32(G)
    state.t += 1
    state.M = momentum_update(state.M, G, hp.beta1, state.m_dtype)
    refreshed = refresh_due(state.t, hp.K)
    if refreshed:
        state.U, state.V = refresh_bases(state.M, state.U, state.V, hp.power_iters)
    recompute = refreshed or not mt_valid
    if state.t == 1:
        state.W, state.v, mt_new, inter = rotated_momentum_apply(state.W, state.v, mt, state.M, G, state.U,
                                                                 state.V, hp.beta1, hp.beta2, hp.eps, hp.lr,
                                                                 recompute=True)
    else:
        state.W, state.v, mt_new, inter = bf16_rotated_momentum_apply(state.W, state.v, mt, state.M, G, state.U,
                                                                      state.V, hp.beta1, hp.beta2, hp.eps, hp.lr,
                                                                      recompute)
    state.last = dict(inter, refreshed=refreshed, bf16=state.t != 1, recompute=recompute)
    return mt_new


# ---- 16-bit storage of the bases --------------------------------------------
#
# [P3] section 3.1 stores the rotation matrices in 16 bits (about 15 % of the
# memory saved). With the bases kept only in bfloat16 the refresh starts from
# the stored values and its result is stored rounded; every step rotates with
# the stored bases, the first one included (there is no binary32 copy to take
# instead).


def refresh_bases_bf16(M, U16, V16, power_iters: int):
    """The refresh of rotated_adam.refresh_bases warm-started from the stored
    16-bit bases (their exact values), the result rounded once to bfloat16."""
    M = np.asarray(M, np.float64)
    m, n = M.shape
    r = min(m, n)
    U = subspace_iteration(M @ M.T, np.asarray(U16, np.float64), r, power_iters)
    V = subspace_iteration(M.T @ M, np.asarray(V16, np.float64), r, power_iters)
    return round_bf16(U), round_bf16(V)


def step_bf16_storage(state: OracleState, G, hp: Hyper) -> OracleState:
    """One step with the bases stored in bfloat16 (state.U, state.V hold
    bfloat16 values): momentum, the refresh from the stored bases when due,
    then bf16_rotation_apply at every step. Mutates and returns ``state``."""
    G = round_f32(G)
    state.t += 1
    state.M = momentum_update(state.M, G, hp.beta1, state.m_dtype)
    refreshed = refresh_due(state.t, hp.K)
    if refreshed:
        state.U, state.V = refresh_bases_bf16(state.M, state.U, state.V, hp.power_iters)
    state.W, state.v, inter = bf16_rotation_apply(state.W, state.v, state.M, G, state.U, state.V, hp.beta2,
                                                  hp.eps, hp.lr)
    state.last = dict(inter, refreshed=refreshed, bf16=True)
    return state
