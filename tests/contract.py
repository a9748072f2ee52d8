"""Teacher-forced parity gates between the device path and the fp64 oracle.

A free-running fp32 trajectory cannot match an fp64 one element by element
on this method, for two reasons intrinsic to it: u = m~ / (sqrt(v) + eps)
turns round-off into O(1/eps) values wherever v is still ~0 (the first step,
the null block after a refresh), and basis columns past the conditioning of
the Gram matrix are determined only up to O(u kappa). So every phase of the
oracle consumes the device's own persisted output of the previous phase and
each gate bounds the error that phase can add:

* Gate M (momentum): oracle EMA of the device's previous M and the same G.
  fp32: max relative error <= 1e-6. bf16: bit-identical except at most
  max(2, 1e-4 n) elements, and every
  element within one bf16 ulp of the reference plus the fp32 rounding of the
  EMA's two terms, 2 u32 (|b1 M| + |(1-b1) G|): the device forms the sum in
  fp32 and rounds once to bf16, the oracle rounds the exact sum; where the
  two terms nearly cancel, their fp32 rounding exceeds one bf16 ulp of the
  small result.
* Gate A (refresh): oracle orthogonal iteration from the device's M and
  previous U, V. (1) orthonormality of the device bases <= 1e-5; (2) forward
  error <= 1e-4 on the well-determined columns, those whose prefix
  conditioning kappa_j = max_{i<=j} 1/|R_ii| of the column-normalised one-shot
  input [(A^p X)[:, :r] | X[:, r:]] is <= 1e2 (or 8 times the error an fp32
  CPU refresh, fp32 products and LAPACK QR, reaches there, if larger: the
  device has measured at up to 5.5 times that reference); the other columns
  are determined only to O(u kappa) and are not compared (several results
  are correct there). Above order 1100, where the oracle's full unblocked QR
  takes minutes, the comparison runs on the leading k = min(r, 256) columns,
  which the oracle forms on their own (the first columns of a QR factor
  depend only on the first columns of its input); (3) the device Q must
  triangularise that input: the strictly lower part of Q^T Z_hat,
  column-normalised, <= 1e-3; (4) the sign convention diag R > 0: every
  diagonal entry of Q^T Z_hat (column-normalised) larger than 1e-2 in
  magnitude is positive (smaller ones are sign-ambiguous at fp32 round-off).
* Gate B16 (the bf16-rotation variant, gate_apply_bf16): as gate B against
  oracle/bf16_rotation.py (the method with U, V rounded to bfloat16, products
  exact); the device's own bf16 roundings of G, M and the intermediates are
  bounded as errors (half an ulp each, the input roundings carried exactly)
  and propagated root-sum-square at 6 sigma.
* Gate MU (the orthogonalised-momentum step, gate_muon): W within
  lr 1e-4 max|O| plus one binary32 rounding of the oracle's Newton-Schulz
  result from the device's M_t.
* Gate B (rotate, moments, apply): oracle from the device's W_{t-1},
  v_{t-1}, M_t, U_t, V_t and the same G. v: max relative error <= 1e-4.
  W elementwise: |W - W_ref| <= tau max|W_ref| + 6 lr sqrt((U.U) E^2 (V.V)^T)
  where E_ab = 4 u32 sqrt(m+n) (rms(m~) + |u_ab| sqrt(1-b2) rms(G~)) /
  (sqrt(v_ab) + eps) is the first-order fp32 error of u propagated
  root-sum-square at 6 sigma; tau = 1e-4 for either storage of M. The
  2e-2 allowed for a bf16 momentum covers its storage rounding, which gate M
  checks; here the oracle reads the device's own stored M, so the rounding
  adds nothing and the fp32 tolerance applies.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List

import numpy as np

import oracle

U32 = 2.0 ** -24


def maxrel(x, ref) -> float:
    ref = np.asarray(ref, np.float64)
    den = np.max(np.abs(ref))
    if den == 0:
        return float(np.max(np.abs(np.asarray(x, np.float64))))
    return float(np.max(np.abs(np.asarray(x, np.float64) - ref)) / den)


@dataclass
class GateReport:
    name: str
    ok: bool
    metrics: Dict[str, float] = field(default_factory=dict)

    def __str__(self):
        ms = ", ".join(f"{k}={v:.3g}" for k, v in self.metrics.items())
        return f"{self.name}: {'ok' if self.ok else 'FAIL'} ({ms})"


def gate_momentum(M_prev, G, M_dev, beta1, m_dtype) -> GateReport:
    ref = oracle.momentum_update(M_prev, G, beta1, m_dtype)
    M_dev = np.asarray(M_dev, np.float64)
    if m_dtype == "f32":
        r = maxrel(M_dev, ref)
        return GateReport("M", r <= 1e-6, {"maxrel": r})
    # The device forms the EMA in fp32 and rounds once to bf16; the oracle
    # rounds the exact value: the two differ by one bf16 ulp only where the
    # fp32 result crosses a rounding boundary (bounded below), and must be
    # identical elsewhere, which catches a wrong rounding mode. A handful of
    # boundary cases is allowed: at most max(2, 1e-4 n) elements.
    differ = int(np.count_nonzero(M_dev != ref))
    b1 = oracle.as_f32_scalar(beta1)
    ulp = np.ldexp(1.0, np.frexp(np.maximum(np.abs(ref), 1e-38))[1] - 8)
    f32_terms = 2 * U32 * (np.abs(b1 * np.asarray(M_prev, np.float64)) + np.abs((1 - b1) * np.asarray(G, np.float64)))
    within = bool(np.all(np.abs(M_dev - ref) <= ulp + f32_terms))
    ok = within and differ <= max(2, int(1e-4 * ref.size))
    return GateReport("M", ok, {"differ": float(differ), "identical": 1.0 - differ / ref.size,
                                "within_bound": float(within)})


def _prefix_kappa(Zhat):
    """Per-column prefix conditioning of the column-normalised matrix."""
    norms = np.linalg.norm(Zhat, axis=0)
    norms[norms == 0] = 1.0
    R = np.linalg.qr(Zhat / norms, mode="r")
    inv = 1.0 / np.maximum(np.abs(np.diag(R)), 1e-300)
    return np.maximum.accumulate(inv)


def one_shot_input(A, X, rank, passes):
    Y = X.copy()
    for _ in range(passes):
        Y = A @ Y
    if rank < X.shape[0]:
        return np.concatenate([Y[:, :rank], X[:, rank:]], axis=1)
    return Y


def fp32_refresh(M_t, X_prev, side, passes):
    """The refresh computed in fp32 on the CPU: Gram products in float32
    (numpy) and a float32 Householder QR (LAPACK sgeqrf through scipy), with
    the same completion and sign convention. Used only to calibrate what an
    fp32 implementation of the refresh attains."""
    import scipy.linalg
    M = np.asarray(M_t, np.float32)
    X = np.asarray(X_prev, np.float32)
    r = min(M.shape)
    for _ in range(passes):
        Y = M @ (M.T @ X[:, :r]) if side == "U" else M.T @ (M @ X[:, :r])
        Z = np.concatenate([Y, X[:, r:]], axis=1).astype(np.float32)
        Q, R = scipy.linalg.qr(Z)
        X = (Q * np.where(np.diag(R) < 0, -1.0, 1.0).astype(np.float32)).astype(np.float32)
    return X.astype(np.float64)


def fp32_refresh_leading(M_t, X_lead, side, passes):
    """fp32_refresh on the leading k <= r columns alone (fp32 Gram products,
    LAPACK sgeqrf on the d x k block), as the oracle's leading-column
    iteration: the fp32 reference of the thin comparison."""
    import scipy.linalg
    M = np.asarray(M_t, np.float32)
    X = np.asarray(X_lead, np.float32)
    for _ in range(passes):
        Y = (M @ (M.T @ X) if side == "U" else M.T @ (M @ X)).astype(np.float32)
        Q, R = scipy.linalg.qr(Y, mode="economic")
        X = (Q * np.where(np.diag(R) < 0, -1.0, 1.0).astype(np.float32)).astype(np.float32)
    return X.astype(np.float64)


# Factor on what an fp32 CPU refresh reaches, for the forward bound. Both
# are fp32 refreshes with different rounding orders (bf16-piece Gram products
# accumulated in K chunks against OpenBLAS sgemm; blocked Householder against
# LAPACK sgeqrf), so their errors on a column are two draws of the same
# O(u kappa_j) quantity and their ratio spreads: the device has measured at
# 0.9 to 5.5 times the reference (the 5.5 on the completed 130 x 130 basis of
# a 130 x 67 matrix refreshed with two passes, where the reference error is
# 1.2e-4); 8 leaves a margin of 1.45 over the largest ratio seen.
FWD_FACTOR = 8.0

# Leading columns compared element by element above the order where the
# oracle's full QR takes minutes.
LEAD_COLS = 256


def _sign_check(Rd_diag):
    """diag R > 0: diagonal entries of Q^T Z_hat (column-normalised) above
    1e-2 in magnitude must be positive; returns (ok, count checked, min)."""
    big = np.abs(Rd_diag) > 1e-2
    return bool(np.all(Rd_diag[big] > 0)), int(big.sum()), float(np.min(Rd_diag[big])) if big.any() else 0.0


def _forward(X_dev_cols, ref, Zhat_cols, ref32):
    """Forward error on the well-determined columns among those given and its
    bound (1e-4, or FWD_FACTOR times what an fp32 reference reaches)."""
    kappa = _prefix_kappa(Zhat_cols)
    good = kappa <= 1e2
    fwd = float(np.max(np.abs(X_dev_cols[:, good] - ref[:, good]))) if good.any() else 0.0
    fwd_tol = 1e-4
    if good.any() and ref32 is not None:
        fwd_tol = max(1e-4, FWD_FACTOR * float(np.max(np.abs(ref32()[:, good] - ref[:, good]))))
    return fwd, fwd_tol, good


def gate_basis(X_dev, A, X_prev, rank, passes, name, forward=True, ref32=None, M_t=None, side=None,
               ref32_lead=None) -> GateReport:
    """forward=False compares only the leading k = min(rank, LEAD_COLS)
    columns with the oracle (for orders where its full unblocked QR takes
    minutes; needs M_t and side), which the oracle forms on their own.
    Orthonormality, triangularisation of the one-shot input and the sign
    convention are checked on the whole basis either way."""
    X_dev = np.asarray(X_dev, np.float64)
    X_prev = np.asarray(X_prev, np.float64)
    d = X_dev.shape[0]
    orth = float(np.max(np.abs(X_dev.T @ X_dev - np.eye(d))))
    Zhat = one_shot_input(A, X_prev, rank, passes)
    if forward:
        ref = oracle.subspace_iteration(A, X_prev, rank, passes)
        # The forward error of an fp32 refresh on these columns grows with the
        # order and the prefix conditioning; near the end of a completed basis
        # the same refresh done in fp32 on the CPU (fp32 Gram products, LAPACK
        # sgeqrf QR) already comes close to 1e-4 (7.5e-5 on a 130 x 130 case).
        fwd, fwd_tol, good = _forward(X_dev, ref, Zhat, ref32)
        ncols = d
    else:
        k = min(rank, LEAD_COLS)
        ref = oracle.leading_subspace_iteration(M_t, X_prev[:, :k], side, passes)
        fwd, fwd_tol, good = _forward(X_dev[:, :k], ref, Zhat[:, :k], ref32_lead)
        ncols = k
    norms = np.linalg.norm(Zhat, axis=0)
    norms[norms == 0] = 1.0
    Rd = X_dev.T @ (Zhat / norms)
    back = float(np.linalg.norm(np.tril(Rd, -1)) / max(np.linalg.norm(Rd), 1e-300))
    sign_ok, nsign, dmin = _sign_check(np.diag(Rd))
    ok = orth <= 1e-5 and fwd <= fwd_tol and back <= 1e-3 and sign_ok
    return GateReport(name, ok, {"orth": orth, "fwd_good": fwd, "fwd_tol": fwd_tol, "fwd_cols": float(ncols),
                                 "good_cols": float(good.sum()), "backward": back, "diag_min": dmin,
                                 "sign_cols": float(nsign)})


def gate_basis_sampled(X_dev, M_t, X_prev, side, passes, name, nsample=256, seed=0) -> GateReport:
    """gate_basis on sampled rows and columns, for orders where the full d^3
    products take minutes on the host: rows S of X^T X - I within 1e-5 of
    zero; below the diagonal in columns C of X^T Z_hat (column-normalised)
    within 1e-3 of their norm, and the diagonal entries of those columns
    positive where they exceed 1e-2; the leading min(r, 256) columns against
    the oracle's leading-column iteration (forward bound as gate_basis). C
    holds the leading r + 8 columns (where the one-shot input is not the
    previous basis) and a random sample. The one-shot input is formed from M
    without building the d x d Gram matrix."""
    X_dev = np.asarray(X_dev, np.float64)
    X_prev = np.asarray(X_prev, np.float64)
    M_t = np.asarray(M_t, np.float64)
    d = X_dev.shape[0]
    r = min(M_t.shape)
    rng = np.random.default_rng(seed)
    pick = lambda extra: np.unique(np.concatenate([extra, rng.choice(d, min(nsample, d), replace=False)]))
    S = pick(np.concatenate([np.arange(min(8, d)), np.arange(max(d - 8, 0), d)]))
    orth = float(np.max(np.abs(X_dev[:, S].T @ X_dev - np.eye(d)[S])))
    Cols = pick(np.arange(min(r + 8, d)))
    Y = X_prev[:, :r]
    for _ in range(passes):
        Y = M_t @ (M_t.T @ Y) if side == "U" else M_t.T @ (M_t @ Y)
    Zc = np.where(Cols[None, :] < r, Y[:, np.minimum(Cols, r - 1)], X_prev[:, Cols])
    norms = np.linalg.norm(Zc, axis=0)
    norms[norms == 0] = 1.0
    Cd = X_dev.T @ (Zc / norms)
    low = np.arange(d)[:, None] > Cols[None, :]
    back = float(np.linalg.norm(Cd[low]) / max(np.linalg.norm(Cd), 1e-300))
    sign_ok, nsign, dmin = _sign_check(Cd[Cols, np.arange(len(Cols))])
    k = min(r, LEAD_COLS)
    ref = oracle.leading_subspace_iteration(M_t, X_prev[:, :k], side, passes)
    fwd, fwd_tol, good = _forward(X_dev[:, :k], ref, Y[:, :k],
                                  lambda: fp32_refresh_leading(M_t, X_prev[:, :k], side, passes))
    ok = orth <= 1e-5 and back <= 1e-3 and sign_ok and fwd <= fwd_tol
    return GateReport(name, ok, {"orth_sampled": orth, "backward_sampled": back, "rows": float(len(S)),
                                 "cols": float(len(Cols)), "diag_min": dmin, "sign_cols": float(nsign),
                                 "fwd_good": fwd, "fwd_tol": fwd_tol, "good_cols": float(good.sum())})


def gate_basis16(X16_dev, M_t, X16_prev, side, passes, name) -> GateReport:
    """A refresh whose result is stored in bfloat16 (bases stored in 16 bits;
    oracle.bf16_rotation.refresh_bases_bf16), teacher-forced from the
    device's previous stored basis. The device rounds its fp32 result, the
    oracle the exact one: on the well-determined columns (prefix conditioning
    <= 1e2, as gate A) each entry within one bf16 ulp of the exact basis plus
    the fp32 forward bound of gate A; orthonormality within 2^-7 (rounding
    each entry by at most 2^-9 relative moves X^T X - I by at most 2^-8);
    the triangularisation of the one-shot input within 1e-2; the sign
    convention as gate A."""
    X = np.asarray(X16_dev, np.float64)
    X0 = np.asarray(X16_prev, np.float64)
    M_t = np.asarray(M_t, np.float64)
    d = X.shape[0]
    r = min(M_t.shape)
    A = M_t @ M_t.T if side == "U" else M_t.T @ M_t
    Zhat = one_shot_input(A, X0, r, passes)
    if d <= 1100:
        ref = oracle.subspace_iteration(A, X0, r, passes)
        ref32 = fp32_refresh(M_t, X0, side, passes)
        kappa = _prefix_kappa(Zhat)
    else:   # the leading columns alone, as gate_basis does at large orders
        k = min(r, LEAD_COLS)
        ref = oracle.leading_subspace_iteration(M_t, X0[:, :k], side, passes)
        ref32 = fp32_refresh_leading(M_t, X0[:, :k], side, passes)
        kappa = _prefix_kappa(Zhat[:, :k])
    good = kappa <= 1e2
    fwd_tol = max(1e-4, FWD_FACTOR * float(np.max(np.abs(ref32[:, good] - ref[:, good])))) if good.any() else 1e-4
    err = np.abs(X[:, :ref.shape[1]][:, good] - ref[:, good])
    ratio = float(np.max(err / (ulp_bf16(ref[:, good]) + fwd_tol))) if good.any() else 0.0   # noqa: E501
    orth = float(np.max(np.abs(X.T @ X - np.eye(d))))
    norms = np.linalg.norm(Zhat, axis=0)
    norms[norms == 0] = 1.0
    Rd = X.T @ (Zhat / norms)
    back = float(np.linalg.norm(np.tril(Rd, -1)) / max(np.linalg.norm(Rd), 1e-300))
    sign_ok, nsign, dmin = _sign_check(np.diag(Rd))
    ok = ratio <= 1.0 and orth <= 2.0 ** -7 and back <= 1e-2 and sign_ok
    return GateReport(name, ok, {"fwd_ratio": ratio, "good_cols": float(good.sum()), "orth": orth,
                                 "backward": back, "diag_min": dmin})


def gate_refresh(M_t, U_prev, V_prev, U_dev, V_dev, passes, forward_max_d=1100) -> List[GateReport]:
    M_t = np.asarray(M_t, np.float64)
    m, n = M_t.shape
    r = min(m, n)
    k = min(r, LEAD_COLS)
    U_prev = np.asarray(U_prev, np.float64)
    V_prev = np.asarray(V_prev, np.float64)
    return [gate_basis(U_dev, M_t @ M_t.T, U_prev, r, passes, "A.U",
                       forward=m <= forward_max_d, ref32=lambda: fp32_refresh(M_t, U_prev, "U", passes),
                       M_t=M_t, side="U",
                       ref32_lead=lambda: fp32_refresh_leading(M_t, U_prev[:, :k], "U", passes)),
            gate_basis(V_dev, M_t.T @ M_t, V_prev, r, passes, "A.V",
                       forward=n <= forward_max_d, ref32=lambda: fp32_refresh(M_t, V_prev, "V", passes),
                       M_t=M_t, side="V",
                       ref32_lead=lambda: fp32_refresh_leading(M_t, V_prev[:, :k], "V", passes))]


def _gate_w_v(W_prev, W_ref, v_ref, it, U_t, V_t, W_dev, v_dev, hp, tau) -> List[GateReport]:
    """v within 1e-4; W element-wise within tau max|W| plus a 6-sigma
    root-sum-square propagation of the first-order fp32 error of u."""
    rv = maxrel(v_dev, v_ref)
    m, n = np.shape(W_prev)
    b2 = oracle.as_f32_scalar(hp.beta2)
    eps = oracle.as_f32_scalar(hp.eps)
    lr = oracle.as_f32_scalar(hp.lr)
    rms = lambda x: float(np.sqrt(np.mean(np.square(x))))
    E = 4 * U32 * np.sqrt(m + n) * (rms(it["mt"]) + np.abs(it["u"]) * np.sqrt(1 - b2) * rms(it["Gt"]))
    E = E / (np.sqrt(v_ref) + eps)
    U = np.asarray(U_t, np.float64)
    V = np.asarray(V_t, np.float64)
    widen = 6.0 * lr * np.sqrt((U * U) @ (E * E) @ (V * V).T)
    base = tau * np.max(np.abs(W_ref))
    err = np.abs(np.asarray(W_dev, np.float64) - W_ref)
    ok_w = bool(np.all(err <= base + widen))
    return [GateReport("B.v", rv <= 1e-4, {"maxrel": rv}),
            GateReport("B.W", ok_w, {"maxrel": maxrel(W_dev, W_ref), "worst_ratio":
                                     float(np.max(err / (base + widen)))})]


def gate_apply(W_prev, v_prev, M_t, G, U_t, V_t, W_dev, v_dev, hp: oracle.Hyper, m_dtype) -> List[GateReport]:
    W_ref, v_ref, it = oracle.rotated_adam_apply(W_prev, v_prev, M_t, G, U_t, V_t, hp.beta2, hp.eps, hp.lr)
    return _gate_w_v(W_prev, W_ref, v_ref, it, U_t, V_t, W_dev, v_dev, hp, 1e-4)


def ulp_bf16(x):
    """One bfloat16 ulp at |x|: 2^(e - 8) for |x| = f 2^e, 0.5 <= f < 1."""
    x = np.abs(np.asarray(x, np.float64))
    return np.ldexp(1.0, np.frexp(np.maximum(x, 2.0 ** -126))[1] - 8)


def gate_apply_bf16(W_prev, v_prev, M_t, G, U_t, V_t, W_dev, v_dev, hp: oracle.Hyper, tau=1e-3,
                    Mt_prev=None, Mt_dev=None, recompute=True) -> List[GateReport]:
    """The bf16-rotation variant (oracle/bf16_rotation.py: the method with U
    and V rounded to bfloat16, every product exact), teacher-forced like
    gate_apply. The device runs the products on bfloat16 operands with
    binary32 accumulation, so it also rounds G (and an fp32 M) and the
    intermediates S = X Vb (X in {G, M}), u and P = u Vb^T to bfloat16; the
    oracle does not. The gate bounds that: each device rounding is at most
    half a bf16 ulp of its value, the known rounding errors of G and M are
    carried through the right rotation exactly (|(rb(X) - X) Vb|), and each
    product adds its binary32 accumulation error 4 u32 sqrt(K); errors are
    propagated root-sum-square through the products (G~ = Ub^T S, P, dW =
    Ub P). Through u the bound is the range of m~ / (sqrt(v) + eps) over G~
    and m~ within 6 times their errors, not a linearisation: bf16 errors are
    large enough that where G~ is below its error (directions where v is
    still tiny) v can fall to b2 v_prev and u jump, and those entries of u
    are determined only up to the rounding (several results are correct
    there). W is bounded element-wise by lr (tau max|dW_ref| + e_dW) +
    2^-23 |W_ref| (one binary32 rounding of W), v by (1 - b2)(2 |G~| e + e^2)
    + 2^-23 |v_ref| + 1e-6 max|v_ref| with e = 6 e_G~.

    With Mt_dev (the carried rotated momentum as well): the oracle is
    bf16_rotated_momentum_apply from the device's Mt_prev; a carried m~ has
    the error (1 - b1) e_G~ of its new term, a recomputed one that of
    Ub^T rb(rb(M) Vb); Mt is bounded by 6 times that plus two binary32
    roundings."""
    from oracle import bf16_rotation as B
    carried = Mt_dev is not None
    if carried:
        W_ref, v_ref, mt_ref, it = B.bf16_rotated_momentum_apply(W_prev, v_prev, Mt_prev, M_t, G, U_t, V_t,
                                                                 hp.beta1, hp.beta2, hp.eps, hp.lr, recompute)
    else:
        W_ref, v_ref, it = B.bf16_rotation_apply(W_prev, v_prev, M_t, G, U_t, V_t, hp.beta2, hp.eps, hp.lr)
    b1 = oracle.as_f32_scalar(hp.beta1)
    b2 = oracle.as_f32_scalar(hp.beta2)
    eps = oracle.as_f32_scalar(hp.eps)
    lr = oracle.as_f32_scalar(hp.lr)
    Ub, Vb = it["Ub"], it["Vb"]
    m, n = Ub.shape[0], Vb.shape[0]
    U2, V2 = Ub * Ub, Vb * Vb
    rss = lambda A2, B2: np.sqrt(A2 @ B2)
    half = lambda x: 0.5 * ulp_bf16(x)

    def right_rotation_error(X, S):
        """Device rb(rb(X) Vb) against the exact X Vb."""
        X = np.asarray(X, np.float64)
        D = oracle.round_bf16(X) - X
        return np.abs(D @ Vb) + half(S) + 4 * U32 * np.sqrt(n) * rss(X * X, V2)

    eSG = right_rotation_error(G, it["SG"])
    eGt = rss(U2.T, eSG ** 2) + 4 * U32 * np.sqrt(m) * rss(U2.T, it["SG"] ** 2)
    if carried and not recompute:
        emt = (1 - b1) * eGt
    else:
        eSM = right_rotation_error(M_t, it["SM"])
        emt = rss(U2.T, eSM ** 2) + 4 * U32 * np.sqrt(m) * rss(U2.T, it["SM"] ** 2)
    u = it["u"]
    # u = m~ / (sqrt(v) + eps) with v = b2 v_prev + (1 - b2) G~^2: the range of
    # u over G~ and m~ within their 6-sigma errors (no linearisation: where
    # G~ is below its bf16 error, v may fall to b2 v_prev and u rise towards
    # m~ / eps, and m~ may change sign), plus the device's rounding of u
    eg, em = 6 * eGt, 6 * emt
    Ga, ma = np.abs(it["Gt"]), np.abs(it["mt"])
    vp = b2 * np.asarray(v_prev, np.float64)
    vmin = vp + (1 - b2) * np.maximum(Ga - eg, 0.0) ** 2
    vmax = vp + (1 - b2) * (Ga + eg) ** 2
    hi = (ma + em) / (np.sqrt(vmin) + eps)
    lo = np.where(ma >= em, (ma - em) / (np.sqrt(vmax) + eps), (ma - em) / (np.sqrt(vmin) + eps))
    ua = np.abs(u)
    Eu = np.maximum(hi - ua, ua - lo) + 6 * half(hi)
    eP = rss(Eu ** 2, V2.T) + 6 * half(it["P"]) + 6 * 4 * U32 * np.sqrt(n) * rss(u ** 2, V2.T)
    edW = rss(U2, eP ** 2) + 6 * 4 * U32 * np.sqrt(m) * rss(U2, it["P"] ** 2)
    bound_w = lr * (tau * np.max(np.abs(it["dW"])) + edW) + 2.0 ** -23 * np.abs(W_ref)
    err_w = np.abs(np.asarray(W_dev, np.float64) - W_ref)
    bound_v = (1 - b2) * (2 * Ga * eg + eg * eg) + 2.0 ** -23 * np.abs(v_ref) + 1e-6 * np.max(v_ref)
    err_v = np.abs(np.asarray(v_dev, np.float64) - v_ref)
    reps = [GateReport("B16.v", bool(np.all(err_v <= bound_v)), {"maxrel": maxrel(v_dev, v_ref),
                                                                 "worst_ratio": float(np.max(err_v / bound_v))}),
            GateReport("B16.W", bool(np.all(err_w <= bound_w)),
                       {"dW_maxrel": float(np.max(err_w) / lr / max(np.max(np.abs(it["dW"])), 1e-300)),
                        "worst_ratio": float(np.max(err_w / bound_w))})]
    if carried:
        bound_m = 6 * emt + 2.0 ** -22 * np.abs(mt_ref) + 1e-30
        err_m = np.abs(np.asarray(Mt_dev, np.float64) - mt_ref)
        reps.insert(0, GateReport("C16.Mt", bool(np.all(err_m <= bound_m)),
                                  {"maxrel": maxrel(Mt_dev, mt_ref), "worst_ratio": float(np.max(err_m / bound_m)),
                                   "recompute": float(recompute)}))
    return reps


def gate_muon(W_prev, M_t, W_dev, hp: oracle.Hyper, iters: int, tau=1e-4) -> GateReport:
    """The orthogonalised-momentum step (oracle/muon.py), teacher-forced from
    the device's M_t and W_{t-1}: |W - W_ref| <= lr tau max|O_ref| +
    2^-23 |W_ref| (tau: the fp32 tolerance, applied to the update itself; one
    binary32 rounding of W). An fp32 emulation of the iteration stays within
    7e-7 of max|O| after 10 iterations."""
    from oracle import muon
    O = muon.newton_schulz_polar(M_t, iters)
    lr = oracle.as_f32_scalar(hp.lr)
    W_ref = oracle.round_f32(np.asarray(W_prev, np.float64) - lr * O)
    err = np.abs(np.asarray(W_dev, np.float64) - W_ref)
    bound = lr * tau * np.max(np.abs(O)) + 2.0 ** -23 * np.abs(W_ref)
    O_dev = (np.asarray(W_prev, np.float64) - np.asarray(W_dev, np.float64)) / lr
    return GateReport("MU.W", bool(np.all(err <= bound)),
                      {"O_maxrel": maxrel(O_dev, O), "worst_ratio": float(np.max(err / bound))})


def gate_apply_rotated_momentum(W_prev, v_prev, Mt_prev, M_t, G, U_t, V_t, W_dev, v_dev, Mt_dev,
                                hp: oracle.Hyper, recompute: bool) -> List[GateReport]:
    """The variant that carries m~ (oracle/rotated_momentum.py): W and v as
    gate_apply with the fp32 tolerance (m~ is carried in fp32 whatever the
    storage of M), and the carried m~ within 1e-5 in Frobenius norm (its fp32
    error is that of one rotation, or of (1 - b1) times one)."""
    from oracle import rotated_momentum as RM
    W_ref, v_ref, mt_ref, it = RM.rotated_momentum_apply(W_prev, v_prev, Mt_prev, M_t, G, U_t, V_t, hp.beta1,
                                                         hp.beta2, hp.eps, hp.lr, recompute)
    d = np.asarray(Mt_dev, np.float64) - mt_ref
    fro = float(np.linalg.norm(d) / max(np.linalg.norm(mt_ref), 1e-300))
    reps = [GateReport("C.Mt", fro <= 1e-5, {"fro_rel": fro, "recompute": float(recompute)})]
    return reps + _gate_w_v(W_prev, W_ref, v_ref, it, U_t, V_t, W_dev, v_dev, hp, 1e-4)
