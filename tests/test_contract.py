"""CPU tests of the parity gates themselves: an honest float32 emulation of
each phase passes, a planted error fails."""

import numpy as np
import torch

import oracle
from tests import contract


def rng(s):
    return np.random.default_rng(s)


def _emulate_momentum_bf16(M, G, b1=0.9):
    b1 = np.float32(b1)
    omb = np.float32(1) - b1
    m32 = (b1 * M.astype(np.float32) + omb * G.astype(np.float32)).astype(np.float32)
    return torch.from_numpy(m32).to(torch.bfloat16).double().numpy()


def test_momentum_gate_bf16_accepts_fp32_rounding_near_cancellation():
    r = rng(0)
    M = oracle.round_bf16(r.standard_normal((256, 256)) * 1e-3)
    G = oracle.round_f32(r.standard_normal((256, 256)) * 1e-3)
    idx = (r.integers(0, 256, 5), r.integers(0, 256, 5))
    G[idx] = oracle.round_f32(-9.0 * M[idx] * (1 + 1e-6))      # b1 M + (1-b1) G ~ 0
    dev = _emulate_momentum_bf16(M, G)
    assert contract.gate_momentum(M, G, dev, 0.9, "bf16").ok
    bad = dev.copy()
    bad[10, 11] = oracle.round_bf16(bad[10, 11] * 1.03)
    assert not contract.gate_momentum(M, G, bad, 0.9, "bf16").ok


def test_momentum_gate_fp32():
    r = rng(1)
    M = oracle.round_f32(r.standard_normal((64, 64)))
    G = oracle.round_f32(r.standard_normal((64, 64)))
    dev = (np.float32(0.9) * M.astype(np.float32) + np.float32(0.1) * G.astype(np.float32)).astype(np.float64)
    assert contract.gate_momentum(M, G, dev, 0.9, "f32").ok
    dev[0, 0] += 1e-4
    assert not contract.gate_momentum(M, G, dev, 0.9, "f32").ok


def test_basis_gate_accepts_fp32_qr_and_rejects_permuted_columns():
    r = rng(2)
    M = r.standard_normal((40, 60)) * 1e-2
    A = M.T @ M
    X0 = np.eye(60)
    Z = contract.one_shot_input(A, X0, 40, 1).astype(np.float32)
    q, rr = np.linalg.qr(Z)                                      # float32 LAPACK
    q = (q * np.where(np.diag(rr) < 0, -1, 1)).astype(np.float64)
    assert contract.gate_basis(q, A, X0, 40, 1, "V").ok
    bad = q.copy()
    bad[:, [0, 1]] = bad[:, [1, 0]]
    assert not contract.gate_basis(bad, A, X0, 40, 1, "V").ok
    flipped = q.copy()
    flipped[:, 2] *= -1                                          # wrong sign convention
    assert not contract.gate_basis(flipped, A, X0, 40, 1, "V").ok


def test_apply_gate_accepts_fp32_emulation_and_rejects_error():
    r = rng(3)
    m, n = 24, 40
    hp = oracle.Hyper()
    W = oracle.round_f32(r.standard_normal((m, n)) * 1e-2)
    v = oracle.round_f32(r.random((m, n)) * 1e-6)
    M = oracle.round_f32(r.standard_normal((m, n)) * 1e-3)
    G = oracle.round_f32(r.standard_normal((m, n)) * 1e-3)
    U = oracle.round_f32(np.linalg.qr(r.standard_normal((m, m)))[0])
    V = oracle.round_f32(np.linalg.qr(r.standard_normal((n, n)))[0])
    f = np.float32
    U32, V32 = U.astype(f), V.astype(f)
    Gt = U32.T @ G.astype(f) @ V32
    mt = U32.T @ M.astype(f) @ V32
    v32 = (f(0.999) * v.astype(f) + f(0.001) * Gt * Gt).astype(f)
    u = mt / (np.sqrt(v32) + f(1e-8))
    W32 = (W.astype(f) - f(1e-3) * (U32 @ u @ V32.T)).astype(np.float64)
    reps = contract.gate_apply(W, v, M, G, U, V, W32, v32.astype(np.float64), hp, "f32")
    assert all(x.ok for x in reps), [str(x) for x in reps]
    bad = W32.copy()
    bad[5, 6] += 3e-4 * np.max(np.abs(W))
    reps = contract.gate_apply(W, v, M, G, U, V, bad, v32.astype(np.float64), hp, "f32")
    assert not all(x.ok for x in reps)


def _emulate_bf16_rotation(W, v, M, G, U, V, hp, transposed_u=False):
    """The bf16-rotation step with binary32 accumulation and the device's
    rounding points, through torch on the CPU (bf16 casts round to nearest
    even)."""
    t = lambda x: torch.from_numpy(np.asarray(x, np.float64)).float()
    bf = lambda x: x.to(torch.bfloat16).float()
    Ub, Vb = bf(t(U)), bf(t(V))
    if transposed_u:
        Ub = Ub.T.contiguous()
    SG = bf(bf(t(G)) @ Vb)
    SM = bf(bf(t(M)) @ Vb)
    Gt = Ub.T @ SG
    mt = Ub.T @ SM
    v32 = np.float32(hp.beta2) * t(v) + (1 - np.float32(hp.beta2)) * Gt * Gt
    u = mt / (torch.sqrt(v32) + np.float32(hp.eps))
    P = bf(bf(u) @ Vb.T)
    W32 = t(W) - np.float32(hp.lr) * (Ub @ P)
    return W32.double().numpy(), v32.double().numpy()


def _bf16_case(seed, m, n):
    r = rng(seed)
    W = oracle.round_f32(r.standard_normal((m, n)) * 1e-2)
    v = oracle.round_f32(r.random((m, n)) * 1e-5)
    M = oracle.round_bf16(r.standard_normal((m, n)) * 1e-3)
    G = oracle.round_f32(r.standard_normal((m, n)) * 1e-2)
    U = oracle.round_f32(np.linalg.qr(r.standard_normal((m, m)))[0])
    V = oracle.round_f32(np.linalg.qr(r.standard_normal((n, n)))[0])
    return W, v, M, G, U, V


def test_bf16_apply_gate_accepts_emulation_and_rejects_errors():
    hp = oracle.Hyper()
    for seed, (m, n) in enumerate([(24, 40), (64, 64), (96, 48)]):
        W, v, M, G, U, V = _bf16_case(10 + seed, m, n)
        Wd, vd = _emulate_bf16_rotation(W, v, M, G, U, V, hp)
        reps = contract.gate_apply_bf16(W, v, M, G, U, V, Wd, vd, hp)
        assert all(x.ok for x in reps), [str(x) for x in reps]
        # a transposed left basis, a 10 % larger step, one corrupted element
        Wt, vt = _emulate_bf16_rotation(W, v, M, G, U, V, hp, transposed_u=True)
        assert not all(x.ok for x in contract.gate_apply_bf16(W, v, M, G, U, V, Wt, vt, hp))
        Wl = oracle.round_f32(W + 1.1 * (Wd - W))
        assert not contract.gate_apply_bf16(W, v, M, G, U, V, Wl, vd, hp)[1].ok
        Wc = Wd.copy()
        Wc[3, 5] -= 0.2 * np.float32(hp.lr) * np.max(np.abs(Wd - W)) / np.float32(hp.lr)
        assert not contract.gate_apply_bf16(W, v, M, G, U, V, Wc, vd, hp)[1].ok


def _emulate_muon(W, M, k, lr, transpose_gram=False):
    X = torch.from_numpy(np.asarray(M, np.float64)).float()
    X = X * (1.0 / torch.sqrt((X.double() ** 2).sum())).float()
    m, n = X.shape
    for _ in range(k):
        wide = (m < n) != transpose_gram
        P = (X @ X.T) @ X if wide else X @ (X.T @ X)
        X = 1.5 * X - 0.5 * P
    return (torch.from_numpy(np.asarray(W, np.float64)).float() - np.float32(lr) * X).double().numpy()


def test_muon_gate_accepts_emulation_and_rejects_errors():
    hp = oracle.Hyper()
    r = rng(20)
    for (m, n) in [(48, 80), (80, 48)]:
        W = oracle.round_f32(r.standard_normal((m, n)) * 1e-2)
        M = oracle.round_bf16(r.standard_normal((m, n)) * 1e-3)
        assert contract.gate_muon(W, M, _emulate_muon(W, M, 5, hp.lr), hp, 5).ok
        assert not contract.gate_muon(W, M, _emulate_muon(W, M, 4, hp.lr), hp, 5).ok          # one step short
        assert not contract.gate_muon(W, M, _emulate_muon(W, M, 5, 1.01 * hp.lr), hp, 5).ok   # lr off by 1 %
        # the Gram matrix of the wrong side is the same iteration: must pass too
        assert contract.gate_muon(W, M, _emulate_muon(W, M, 5, hp.lr, transpose_gram=True), hp, 5).ok


def test_sampled_basis_gate_accepts_lapack_and_rejects_swaps():
    r = rng(30)
    M = r.standard_normal((200, 12)) * 1e-2
    X0 = np.eye(200)
    Z = contract.one_shot_input(M @ M.T, X0, 12, 1)
    q, rr = np.linalg.qr(Z.astype(np.float32))
    q = (q * np.where(np.diag(rr) < 0, -1, 1)).astype(np.float64)
    assert contract.gate_basis_sampled(q, M, X0, "U", 1, "U", nsample=64).ok
    bad = q.copy()
    bad[:, [3, 150]] = bad[:, [150, 3]]                       # a completion column moved into the leading block
    assert not contract.gate_basis_sampled(bad, M, X0, "U", 1, "U", nsample=64).ok
    skew = q.copy()
    skew[:, 5] += 1e-3 * skew[:, 6]                           # not orthonormal
    assert not contract.gate_basis_sampled(skew, M, X0, "U", 1, "U", nsample=64).ok


def test_basis_gate_at_large_orders_compares_leading_columns_and_signs(monkeypatch):
    """forward=False (orders where the oracle's full QR takes minutes): the
    leading columns are compared with the oracle's leading-column iteration,
    and the sign convention is checked on the whole basis. A fp32 LAPACK
    refresh passes; a perturbed leading column and a flipped completion
    column fail."""
    monkeypatch.setattr(contract, "LEAD_COLS", 32)
    r = rng(40)
    M = r.standard_normal((300, 120)) * 1e-2
    X0 = contract.fp32_refresh(M, np.eye(300), "U", 1)         # a warm, non-identity start
    q = contract.fp32_refresh(M, X0, "U", 2)
    gate = lambda X: contract.gate_refresh(M, X0, np.eye(120), X, contract.fp32_refresh(M, np.eye(120), "V", 2),
                                           2, forward_max_d=100)
    reps = gate(q)
    assert all(x.ok for x in reps), [str(x) for x in reps]
    assert reps[0].metrics["fwd_cols"] == 32 and reps[0].metrics["good_cols"] > 0
    bad = q.copy()
    bad[:, 3] += 1e-3 * bad[:, 4]
    assert not gate(bad)[0].ok
    flipped = q.copy()
    flipped[:, 250] *= -1                                          # a completion column with the wrong sign
    rep = gate(flipped)[0]
    assert not rep.ok and rep.metrics["orth"] <= 1e-5 and rep.metrics["fwd_good"] <= rep.metrics["fwd_tol"]


def test_sampled_basis_gate_rejects_a_flipped_sign():
    r = rng(31)
    M = r.standard_normal((200, 12)) * 1e-2
    X0 = np.eye(200)
    Z = contract.one_shot_input(M @ M.T, X0, 12, 1)
    q, rr = np.linalg.qr(Z.astype(np.float32))
    q = (q * np.where(np.diag(rr) < 0, -1, 1)).astype(np.float64)
    flipped = q.copy()
    flipped[:, 5] *= -1                                            # leading block: also the forward check
    assert not contract.gate_basis_sampled(flipped, M, X0, "U", 1, "U", nsample=64).ok
    flipped = q.copy()
    flipped[:, 13] *= -1                                           # first completion column (always sampled)
    rep = contract.gate_basis_sampled(flipped, M, X0, "U", 1, "U", nsample=64)
    assert not rep.ok and rep.metrics["diag_min"] < 0


def test_apply_gate_holds_a_bf16_momentum_to_the_fp32_tolerance():
    """The oracle reads the device's stored bf16 M, so the rotations see the
    same values and the fp32 tolerance applies: an fp32 emulation passes and
    a 1e-3 relative error of the update (inside the old 2e-2 allowance)
    fails."""
    r = rng(33)
    m, n = 24, 40
    hp = oracle.Hyper()
    W = oracle.round_f32(r.standard_normal((m, n)) * 1e-2)
    v = oracle.round_f32(r.random((m, n)) * 1e-6)
    M = oracle.round_bf16(r.standard_normal((m, n)) * 1e-3)
    G = oracle.round_f32(r.standard_normal((m, n)) * 1e-3)
    U = oracle.round_f32(np.linalg.qr(r.standard_normal((m, m)))[0])
    V = oracle.round_f32(np.linalg.qr(r.standard_normal((n, n)))[0])
    f = np.float32
    U32, V32 = U.astype(f), V.astype(f)
    Gt = U32.T @ G.astype(f) @ V32
    mt = U32.T @ M.astype(f) @ V32
    v32 = (f(0.999) * v.astype(f) + f(0.001) * Gt * Gt).astype(f)
    u = mt / (np.sqrt(v32) + f(1e-8))
    dW = (U32 @ u @ V32.T).astype(np.float64)
    W32 = oracle.round_f32(W - f(1e-3) * dW)
    assert all(x.ok for x in contract.gate_apply(W, v, M, G, U, V, W32, v32.astype(np.float64), hp, "bf16"))
    off = oracle.round_f32(W - f(1e-3) * dW * (1 + 1e-3))
    assert not all(x.ok for x in contract.gate_apply(W, v, M, G, U, V, off, v32.astype(np.float64), hp, "bf16"))
