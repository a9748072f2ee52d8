"""Plain CPU oracle of the optimizer-state health checks and of the basis
re-orthonormalisation (float64).

TEST INFRASTRUCTURE. Only ``tests/`` may import or call this module; the
library's ``opt_group_health`` and ``opt_group_reorthonormalize`` share no
code with it.

Sources, cited by page title and section:

* [P3] "Pipeline parallelism and gradient staleness optimisation in
  distributed training", section 5.1: when training oscillates, check that
  the rotation matrices are orthogonal (U^T U = I), and restore
  orthogonality with U (U^T U)^(-1/2) (the printed line is garbled: the
  product operator is lost and the inverse square root is written as an
  elementwise square root of the inverse; the reading taken is the matrix
  inverse square root, the symmetric (Loewdin) orthonormalisation, which is
  the polar factor of U).
* [P2] "Large-model distributed optimisation: three-layer decoupling of
  communication, memory and compute", section 4.3: a ratio
  std(v) / mean(|v|) above 10 flags a contaminated second moment; section
  4.4: watch the minimum of v (it must stay positive where it divides).

Definitions used here (each listed in the design doc): orthogonality drift is the
largest absolute entry of X^T X - I; std is the population standard
deviation; non-finite counts NaN and +-Inf entries of W, M and v.
"""

from __future__ import annotations

import numpy as np

__all__ = ["orth_drift", "v_stats", "nonfinite", "polar_factor", "newton_schulz"]


def orth_drift(X) -> float:
    """max_ij |(X^T X - I)_ij| of a square basis, in float64."""
    X = np.asarray(X, np.float64)
    return float(np.max(np.abs(X.T @ X - np.eye(X.shape[1]))))


def v_stats(v):
    """(mean |v|, std v, min v, max v) over the finite and non-finite entries
    alike (a NaN propagates)."""
    v = np.asarray(v, np.float64).ravel()
    mean = v.mean()
    return float(np.abs(v).mean()), float(np.sqrt(np.mean((v - mean) ** 2))), float(v.min()), float(v.max())


def nonfinite(*arrays) -> int:
    return int(sum(np.count_nonzero(~np.isfinite(np.asarray(a, np.float64))) for a in arrays))


def polar_factor(X):
    """X (X^T X)^(-1/2) through the eigendecomposition of X^T X ([P3] 5.1)."""
    X = np.asarray(X, np.float64)
    w, Q = np.linalg.eigh(X.T @ X)
    return X @ (Q * (1.0 / np.sqrt(w))) @ Q.T


def newton_schulz(X, iters: int):
    """iters steps of X <- X (3 I - X^T X) / 2, the iteration that converges
    quadratically to the polar factor when ||X^T X - I||_2 < 1."""
    X = np.asarray(X, np.float64)
    I = np.eye(X.shape[1])
    for _ in range(iters):
        X = X @ (1.5 * I - 0.5 * (X.T @ X))
    return X
