"""Plain fp64 CPU oracle of the rotated-basis matrix-optimizer step.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module. The HIP
product path never routes through it, and it shares no code with that path.

Everything here is numpy float64 with library matrix products as the only
primitives. Storage rounding (binary32 or bfloat16, round-to-nearest-even) is
applied exactly where the device path stores persistent state, so that a
teacher-forced comparison sees the same quantisation points.

Sources, cited by page title and section (the pages are scraped web text):

* [P3] "Pipeline parallelism and gradient staleness optimisation in
  distributed training" (mhpn.cn):
  - section 2.1: the per-coordinate Adam update divides the first moment by
    the square root of the second moment plus eps, then subtracts lr times
    that quotient from the parameter; no bias correction appears.
  - section 2.2: a momentum matrix M of the same m x n shape as each weight
    matrix W; every K iterations a power iteration with a QR factorisation
    yields a left basis from M and a right basis from M transposed; the
    two-sided rotation is U^T (.) V.
  - section 4.2: rotation frequency of every 10 iterations (<=7B) or 5 (>7B).
  - section 5.1: the bases must satisfy U^T U = I.
* [P2] "Large-model distributed optimisation: three-layer decoupling of
  communication, memory and compute" (sheratonhq.com):
  - section 2.1: second-moment recurrence v = beta2 v + (1 - beta2) g^2.
  - section 2.2: first moment as an exponential moving average with weight
    beta1 on the old value (used here for M).
  - section 3.3: first moment kept in bfloat16, second moment and master
    weights in float32.
  - section 5.2: the gradient is squared in float32 before entering v.

Readings where the pages are silent or garbled (each listed in the design doc):
the momentum is the EMA M <- b1 M + (1-b1) G; inside one step the order is
momentum -> refresh (when due, from the new M) -> rotate -> moments -> apply;
the refresh is due at t = 1, K+1, 2K+1, ... (t counts from 1; K = 0 never);
the power iteration is a full-basis orthogonal iteration warm-started from the
current basis with one Gram multiplication and one QR per pass; the QR sign
convention is diag(R) > 0 (a zero diagonal counts as positive); for m != n the
larger Gram matrix has rank r = min(m, n) and its trailing columns are
completed from the previous basis, Z = [Y[:, :r] | X[:, r:]]; the initial bases
are identities supplied by the caller; v is not re-projected when the basis
changes.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "BF16_MAX",
    "round_f32",
    "round_bf16",
    "store",
    "as_f32_scalar",
    "Hyper",
    "OracleState",
    "momentum_update",
    "householder_qr",
    "orthonormal_factor",
    "subspace_iteration",
    "leading_subspace_iteration",
    "refresh_bases",
    "rotated_adam_apply",
    "refresh_due",
    "step",
]

# Largest finite bfloat16: (2 - 2^-7) * 2^127.
BF16_MAX = (2.0 - 2.0 ** -7) * 2.0 ** 127


def round_f32(x):
    """Round every element to the nearest binary32 value (ties to even).

    The result is returned as float64 holding exactly the binary32 values.
    """
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def round_bf16(x):
    """Round every element to the nearest bfloat16 value, ties to even.

    bfloat16 keeps 8 significant bits and the binary32 exponent range, so a
    finite x = f * 2^e (0.5 <= |f| < 1) is quantised to a multiple of
    2^(e - 8); below the normal range (e < -125) the quantum stays 2^-133.
    Values whose rounding exceeds the largest finite bfloat16 become +-inf.
    NaN and +-inf pass through unchanged.
    """
    x = np.asarray(x, dtype=np.float64)
    out = x.copy()
    fin = np.isfinite(x)
    xf = x[fin]
    _, e = np.frexp(xf)
    quantum = np.ldexp(1.0, np.maximum(e, -125) - 8)
    r = np.rint(xf / quantum) * quantum  # scaling by a power of two is exact
    over = np.abs(r) > BF16_MAX
    r[over] = np.copysign(np.inf, xf[over])
    out[fin] = r
    return out


def store(x, dtype: str):
    """Quantise to the storage type of a persistent tensor ('f32' or 'bf16')."""
    if dtype == "f32":
        return round_f32(x)
    if dtype == "bf16":
        return round_bf16(x)
    raise ValueError(f"unknown storage dtype {dtype!r}")


def as_f32_scalar(x: float) -> float:
    """The binary32 value of a hyper-parameter, as the device receives it."""
    return float(np.float32(x))


@dataclass(frozen=True)
class Hyper:
    beta1: float = 0.9
    beta2: float = 0.999
    eps: float = 1e-8
    lr: float = 1e-3
    K: int = 10            # refresh period; 0 disables automatic refreshes
    power_iters: int = 1   # orthogonal-iteration passes per refresh


@dataclass
class OracleState:
    """Persistent per-matrix state, every array float64 holding stored values."""

    W: np.ndarray
    M: np.ndarray
    v: np.ndarray
    U: np.ndarray
    V: np.ndarray
    m_dtype: str = "f32"
    t: int = 0
    last: dict = field(default_factory=dict)

    @classmethod
    def fresh(cls, W0, m_dtype: str = "f32") -> "OracleState":
        """Zero moments and identity bases, the caller-side initial state."""
        W0 = round_f32(W0)
        m, n = W0.shape
        return cls(W=W0, M=np.zeros((m, n)), v=np.zeros((m, n)),
                   U=np.eye(m), V=np.eye(n), m_dtype=m_dtype)


def momentum_update(M, G, beta1: float, m_dtype: str):
    """Momentum matrix as an exponential moving average of the gradient.

    [P3] section 2.2 keeps one momentum matrix per weight matrix; [P2] section
    2.2 gives the EMA form with weight beta1 on the previous value. The sum
    is exact in float64 and rounded once to the storage type of M.
    """
    b1 = as_f32_scalar(beta1)
    return store(b1 * np.asarray(M, np.float64) + (1.0 - b1) * np.asarray(G, np.float64),
                 m_dtype)


def householder_qr(Z, q_cols=None):
    """Unblocked Householder QR of a square or tall matrix: Z = Q R.

    Column j is reduced by the reflector H_j = I - tau_j v_j v_j^T with
    v_j[0] = 1, chosen as in the textbook construction: beta = -sign(alpha)
    * ||x||, tau = (beta - alpha) / beta, v = x / (alpha - beta). A column
    whose part below the diagonal is exactly zero takes tau = 0 (H_j = I)
    and keeps its diagonal entry. Q is accumulated explicitly by applying
    the reflectors to the identity in reverse order.

    Returns (Q, R) with Q of shape (rows, rows) and R of shape (rows, cols).
    With q_cols = k (at most cols) only the leading k columns of Q are
    formed, the reflectors applied to the first k columns of the identity:
    Q is then rows x k. Q[:, j] = H_0 ... H_j e_j depends only on the
    reflectors of columns 0..j, so these are the leading columns of the
    full Q.
    """
    A = np.array(Z, dtype=np.float64, copy=True)
    rows, cols = A.shape
    if rows < cols:
        raise ValueError("householder_qr expects rows >= cols")
    reflectors = []
    for j in range(cols):
        x = A[j:, j]
        alpha = x[0]
        sigma = float(x[1:] @ x[1:])
        if sigma == 0.0:
            reflectors.append((None, 0.0))
            continue
        norm = math.sqrt(alpha * alpha + sigma)
        beta = -math.copysign(norm, alpha)
        v = x / (alpha - beta)
        v[0] = 1.0
        tau = (beta - alpha) / beta
        w = v @ A[j:, j:]
        A[j:, j:] -= tau * np.outer(v, w)
        A[j + 1:, j] = 0.0
        A[j, j] = beta
        reflectors.append((v, tau))
    k = rows if q_cols is None else q_cols
    if k > rows or (q_cols is not None and k > cols):
        raise ValueError("q_cols must not exceed the column count")
    Q = np.eye(rows, k)
    for j in range(min(cols, k) - 1, -1, -1):
        v, tau = reflectors[j]
        if v is None:
            continue
        w = v @ Q[j:, j:]
        Q[j:, j:] -= tau * np.outer(v, w)
    return Q, np.triu(A)


def orthonormal_factor(Z, q_cols=None):
    """The Q factor of Z = QR normalised so that diag(R) > 0.

    A zero diagonal entry of R counts as positive. For a full-rank square Z
    this Q is unique, whatever reflector convention produced it. With
    q_cols = k only its leading k columns are formed (householder_qr).
    """
    Q, R = householder_qr(Z, q_cols)
    signs = np.where(np.diag(R)[:Q.shape[1]] < 0.0, -1.0, 1.0)
    return Q * signs[np.newaxis, :]


def leading_subspace_iteration(M, X_lead, side: str, passes: int):
    """The leading k columns of subspace_iteration for the left (side 'U',
    A = M M^T) or right ('V', A = M^T M) basis of M, for k <= r = min(m, n):
    the first k columns of a QR factor depend only on the first k columns of
    its input, and those of A X depend only on those of X, so each pass is
    Y = A X_lead (formed as M (M^T X_lead) or M^T (M X_lead)) followed by the
    leading k columns of the positive-diagonal QR of Y. Exactly the
    iteration's arithmetic restricted to those columns (no completion is
    needed below the rank)."""
    M = np.asarray(M, np.float64)
    X = np.asarray(X_lead, np.float64)
    if X.shape[1] > min(M.shape):
        raise ValueError("leading_subspace_iteration needs k <= min(m, n)")
    for _ in range(passes):
        Y = M @ (M.T @ X) if side == "U" else M.T @ (M @ X)
        X = orthonormal_factor(Y, q_cols=Y.shape[1])
    return X


def subspace_iteration(A, X, rank: int, passes: int):
    """Orthogonal iteration on the symmetric matrix A, warm-started at X.

    Each pass multiplies by A once and re-orthonormalises with a
    positive-diagonal QR. When A has rank r smaller than its order, only the
    leading r columns of the product carry information; the trailing columns
    of the QR input are taken from the current basis, Z = [Y[:, :r] | X[:, r:]],
    so the completion is a Gram-Schmidt continuation of the previous basis.
    """
    d = X.shape[0]
    X = np.asarray(X, np.float64)
    for _ in range(passes):
        Y = A @ X
        if rank < d:
            Z = np.concatenate([Y[:, :rank], X[:, rank:]], axis=1)
        else:
            Z = Y
        X = orthonormal_factor(Z)
    return X


def refresh_bases(M, U, V, power_iters: int):
    """Left and right bases from the momentum matrix ([P3] section 2.2).

    U spans the eigenvectors of M M^T (left singular vectors of M), V those of
    M^T M (right singular vectors). Both are stored as binary32.
    """
    M = np.asarray(M, np.float64)
    m, n = M.shape
    r = min(m, n)
    U_new = subspace_iteration(M @ M.T, U, r, power_iters)
    V_new = subspace_iteration(M.T @ M, V, r, power_iters)
    return round_f32(U_new), round_f32(V_new)


def rotated_adam_apply(W, v, M, G, U, V, beta2: float, eps: float, lr: float):
    """Rotate into the basis, run Adam moments there, rotate back and apply.

    G~ = U^T G V and m~ = U^T M V ([P3] section 2.2); v <- b2 v + (1-b2) G~^2
    with G~ squared at full precision ([P2] sections 2.1 and 5.2);
    u = m~ / (sqrt(v) + eps) and W <- W - lr U u V^T ([P3] section 2.1, no bias
    correction). v and W are stored as binary32; u uses the stored v.

    Returns (W_new, v_new, intermediates) where intermediates holds Gt, mt, u
    and dW = U u V^T in float64.
    """
    b2 = as_f32_scalar(beta2)
    eps = as_f32_scalar(eps)
    lr = as_f32_scalar(lr)
    U = np.asarray(U, np.float64)
    V = np.asarray(V, np.float64)
    Gt = U.T @ np.asarray(G, np.float64) @ V
    mt = U.T @ np.asarray(M, np.float64) @ V
    v_new = round_f32(b2 * np.asarray(v, np.float64) + (1.0 - b2) * (Gt * Gt))
    u = mt / (np.sqrt(v_new) + eps)
    dW = U @ u @ V.T
    W_new = round_f32(np.asarray(W, np.float64) - lr * dW)
    return W_new, v_new, {"Gt": Gt, "mt": mt, "u": u, "dW": dW}


def refresh_due(t: int, K: int) -> bool:
    """Refresh at t = 1, K+1, 2K+1, ... (t counts steps from 1); K = 0: never."""
    return K > 0 and (t - 1) % K == 0


def step(state: OracleState, G, hp: Hyper) -> OracleState:
    """One optimizer step on one matrix, in the order momentum -> refresh ->
    rotate -> moments -> apply. Mutates and returns ``state``."""
    G = round_f32(G)
    state.t += 1
    state.M = momentum_update(state.M, G, hp.beta1, state.m_dtype)
    refreshed = refresh_due(state.t, hp.K)
    if refreshed:
        state.U, state.V = refresh_bases(state.M, state.U, state.V, hp.power_iters)
    state.W, state.v, inter = rotated_adam_apply(
        state.W, state.v, state.M, G, state.U, state.V, hp.beta2, hp.eps, hp.lr)
    state.last = dict(inter, refreshed=refreshed)
    return state
