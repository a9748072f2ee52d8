"""Plain fp64 CPU oracle of the orthogonalised-momentum update (a Muon-style
matrix optimizer step).

TEST INFRASTRUCTURE. Only ``tests/`` and ``__graft_entry__.smoke()`` may
import or call this module; it shares no code with the HIP path.

The Canzona page (aitangshan.cn), section 1 and section 7 (extended
applications), names Muon among the matrix optimizers the framework runs and credits it with
a faster orthogonalisation step; the pages give no formula. Readings, each
the plainest one the rest supports:

* the momentum is the same EMA as the rotated method's ([P2] "Large-model
  distributed optimisation: three-layer decoupling of communication, memory
  and compute", section 2.2), stored fp32 or bf16;
* the orthogonalisation replaces M by its orthogonal polar factor O (the
  nearest matrix with orthonormal rows or columns: O = P Q^T for the thin SVD
  M = P S Q^T), approximated by the textbook cubic Newton-Schulz iteration
  X <- 1.5 X - 0.5 X X^T X from X_0 = M / ||M||_F (singular values in
  (0, 1], so every one converges to 1), run for a fixed number of
  iterations on the side whose Gram matrix is smaller;
* the update is W <- W - lr O (no extra scaling), W stored binary32.

The iteration is the definition here (a fixed iteration count approximates
the polar factor); the polar factor itself pins it (test_muon_oracle.py).
"""

from __future__ import annotations

import numpy as np

from .rotated_adam import as_f32_scalar, momentum_update, round_f32

__all__ = ["newton_schulz_polar", "polar_factor_svd", "muon_apply"]


def newton_schulz_polar(M, iters: int):
    """X_0 = M / ||M||_F, then `iters` steps X <- 1.5 X - 0.5 X X^T X (for
    m >= n; for m < n the transposed form X <- 1.5 X - 0.5 X X^T X is taken
    with the m x m Gram matrix X X^T on the left, which is the same
    iteration). A zero matrix stays zero."""
    X = np.asarray(M, np.float64)
    nrm = np.linalg.norm(X)
    if nrm == 0.0:
        return np.zeros_like(X)
    X = X / nrm
    m, n = X.shape
    for _ in range(iters):
        if m >= n:
            X = 1.5 * X - 0.5 * (X @ (X.T @ X))
        else:
            X = 1.5 * X - 0.5 * ((X @ X.T) @ X)
    return X


def polar_factor_svd(M):
    """The orthogonal polar factor P Q^T of the thin SVD M = P S Q^T."""
    P, _, Qt = np.linalg.svd(np.asarray(M, np.float64), full_matrices=False)
    return P @ Qt


def muon_apply(W, M, G, beta1: float, lr: float, iters: int, m_dtype: str):
    """One step: M <- EMA (stored in m_dtype), O = newton_schulz_polar(M),
    W <- rf(W - lr O). Returns (W_new, M_new, O)."""
    M_new = momentum_update(M, round_f32(G), beta1, m_dtype)
    O = newton_schulz_polar(M_new, iters)
    W_new = round_f32(np.asarray(W, np.float64) - as_f32_scalar(lr) * O)
    return W_new, M_new, O
