"""GPU tests of the building blocks, called through the C ABI.

GEMM: every operand variant against float64 products of the same fp32/bf16
inputs, with an element-wise bound K * 2^-23 * (|A| |B|)_ij (the standard
forward error bound of an fp32 dot product, doubled).
QR: against the oracle's positive-diagonal orthonormal factor on well
conditioned inputs, and through size-independent properties on Gaussian ones.
"""

import numpy as np
import pytest

pytestmark = pytest.mark.gpu


def _torch():
    import torch
    return torch


def _mo():
    import matrix_optimizer_step_02_amd as mo
    return mo


def _gemm_case(ta, tb, a_bf16, b_bf16, M, N, K, alpha=1.0, beta=0.0, seed=0, x6=False):
    torch = _torch()
    mo = _mo()
    N_ = mo.native
    g = torch.Generator(device="cuda").manual_seed(seed)
    ashape = (K, M) if ta else (M, K)
    bshape = (N, K) if tb else (K, N)
    A = torch.randn(*ashape, generator=g, device="cuda")
    B = torch.randn(*bshape, generator=g, device="cuda")
    if a_bf16:
        A = A.to(torch.bfloat16)
    if b_bf16:
        B = B.to(torch.bfloat16)
    C = torch.randn(M, N, generator=g, device="cuda")
    C0 = C.double().cpu().numpy()
    lda = ashape[1]
    ldb = bshape[1]
    (N_.opt_gemm_x6 if x6 else N_.opt_gemm)(ta, tb, M, N, K, alpha, A.data_ptr(), int(a_bf16), lda, B.data_ptr(),
                                             int(b_bf16), ldb, beta, C.data_ptr(), N, mo.stream_ptr())
    torch.cuda.synchronize()
    An = A.double().cpu().numpy()
    Bn = B.double().cpu().numpy()
    opA = An.T if ta else An
    opB = Bn.T if tb else Bn
    ref = alpha * (opA @ opB) + beta * C0
    bound = 2 * max(K, 1) * 2.0 ** -23 * (np.abs(alpha) * (np.abs(opA) @ np.abs(opB)) + np.abs(beta * C0)) + 1e-30
    err = np.abs(C.double().cpu().numpy() - ref)
    return float(np.max(err / bound))


@pytest.mark.parametrize("ta,tb,a_bf16,b_bf16", [(0, 0, 0, 0), (1, 0, 0, 0), (0, 1, 0, 0), (0, 0, 0, 1), (0, 0, 1, 0),
                                                  (1, 0, 1, 0)])
def test_gemm_x6_variants(ta, tb, a_bf16, b_bf16):
    """fp32 products on bf16 MFMAs (three-piece split, six piece products):
    the fp32 dot-product bound holds element by element (the terms left out
    add at most 2^-23 (|A| |B|)_ij), on ragged shapes, k tails shorter than
    a 16-deep MFMA step, both tile configurations and beta != 0."""
    print(f"gemm_x6 ta={ta} tb={tb} abf={a_bf16} bbf={b_bf16}", flush=True)
    for (M, N, K) in [(130, 67, 45), (256, 384, 512), (1, 1, 1), (33, 129, 3), (200, 300, 1000),
                      (4096, 2048, 200), (8192, 4100, 300)]:   # the last one on 256 x 256 tiles
        r = _gemm_case(ta, tb, a_bf16, b_bf16, M, N, K, alpha=-0.75, beta=0.5, x6=True)
        print(f"  {M}x{N}x{K}: worst err/bound {r:.3f}", flush=True)
        assert r <= 1.0, (M, N, K, r)


def test_gemm_x6_rejects_other_layouts():
    import matrix_optimizer_step_02_amd as mo
    torch = _torch()
    A = torch.zeros(8, 8, device="cuda")
    C = torch.zeros(8, 8, device="cuda")
    with pytest.raises(mo.MatoptError):
        mo.native.opt_gemm_x6(1, 1, 8, 8, 8, 1.0, A.data_ptr(), 0, 8, A.data_ptr(), 0, 8, 0.0, C.data_ptr(), 8,
                              mo.stream_ptr())


@pytest.mark.parametrize("ta,tb", [(0, 0), (1, 0), (0, 1), (1, 1)])
@pytest.mark.parametrize("a_bf16,b_bf16", [(0, 0), (1, 0), (0, 1)])
def test_gemm_variants_ragged(ta, tb, a_bf16, b_bf16):
    print(f"gemm ta={ta} tb={tb} abf={a_bf16} bbf={b_bf16}", flush=True)
    for (M, N, K) in [(130, 67, 45), (256, 384, 512), (1, 1, 1), (33, 129, 3), (200, 300, 1000)]:
        r = _gemm_case(ta, tb, a_bf16, b_bf16, M, N, K, alpha=0.75, beta=0.5)
        assert r <= 1.0, (M, N, K, r)


def test_gemm_empty_k_scales_c():
    r = _gemm_case(0, 0, 0, 0, 70, 90, 0, alpha=1.0, beta=2.0)
    assert r <= 1.0


def test_gemm_large_square():
    print("gemm 2048^3", flush=True)
    r = _gemm_case(1, 0, 0, 0, 2048, 2048, 2048)
    assert r <= 1.0


def _orthonormalize(Z):
    torch = _torch()
    mo = _mo()
    N_ = mo.native
    d = Z.shape[0]
    Zd = torch.tensor(Z, dtype=torch.float32, device="cuda").contiguous()
    Q = torch.empty_like(Zd)
    ws_bytes = N_.opt_orthonormalize_workspace_size(d)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    N_.opt_orthonormalize(Zd.data_ptr(), Q.data_ptr(), d, ws.data_ptr(), ws_bytes, mo.stream_ptr())
    torch.cuda.synchronize()
    return Q.double().cpu().numpy()


@pytest.mark.parametrize("d", [1, 2, 5, 31, 32, 33, 64, 100, 257, 512])
def test_orthonormalize_well_conditioned_matches_oracle(d):
    import oracle
    print(f"qr d={d}", flush=True)
    rng = np.random.default_rng(d)
    Z = np.eye(d) + 0.3 * rng.standard_normal((d, d)) / np.sqrt(d)
    Z = oracle.round_f32(Z)
    Q = _orthonormalize(Z)
    ref = oracle.orthonormal_factor(Z)
    assert np.max(np.abs(Q - ref)) < 2e-5
    assert np.max(np.abs(Q.T @ Q - np.eye(d))) < 1e-5


@pytest.mark.parametrize("d", [6400, 8200])
def test_orthonormalize_tall_panels_match_oracle(d):
    """Panels of more than 6144 rows are factorised on the tall path (the
    panel's rows spread over resident workgroups, one cooperative launch, a
    grid-wide barrier per column). Well-conditioned input; the leading 320
    columns of Q (which depend only on the leading columns of Z) against the
    oracle's positive-diagonal factor of those columns, and the whole Q's
    orthonormality."""
    import oracle
    print(f"qr tall d={d}", flush=True)
    rng = np.random.default_rng(d)
    Z = oracle.round_f32(np.eye(d) + 0.3 * rng.standard_normal((d, d)) / np.sqrt(d))
    Q = _orthonormalize(Z)
    k = 320
    ref = oracle.orthonormal_factor(Z[:, :k], q_cols=k)
    assert np.max(np.abs(Q[:, :k] - ref)) < 2e-5
    assert np.max(np.abs(Q.T @ Q - np.eye(d))) < 1e-5
    # the cross-workgroup sums are added in a fixed slice order: a second
    # factorisation of the same input is bitwise the same
    assert np.array_equal(_orthonormalize(Z), Q)


@pytest.mark.parametrize("d", [64, 300, 1024, 2500])
def test_orthonormalize_gaussian_properties(d):
    print(f"qr gauss d={d}", flush=True)
    rng = np.random.default_rng(100 + d)
    Z = rng.standard_normal((d, d)).astype(np.float32).astype(np.float64)
    Q = _orthonormalize(Z)
    assert np.max(np.abs(Q.T @ Q - np.eye(d))) < 1e-5
    R = Q.T @ Z
    assert np.linalg.norm(np.tril(R, -1)) <= 1e-5 * np.linalg.norm(Z)
    assert np.all(np.diag(R) > 0)


def test_orthonormalize_zero_and_rank_deficient():
    Q = _orthonormalize(np.zeros((40, 40)))
    assert np.array_equal(Q, np.eye(40))
    rng = np.random.default_rng(7)
    Z = rng.standard_normal((70, 70))
    Z[:, 10:20] = 0.0
    Z[:, 30] = Z[:, 5]
    Z = Z.astype(np.float32).astype(np.float64)
    Q = _orthonormalize(Z)
    assert np.max(np.abs(Q.T @ Q - np.eye(70))) < 1e-5
    R = Q.T @ Z
    assert np.linalg.norm(np.tril(R, -1)) <= 1e-5 * np.linalg.norm(Z)


@pytest.mark.parametrize("ta,tb,b_bf16", [(0, 0, 0), (1, 0, 1), (0, 1, 0)])
def test_gemm_large_tile_configuration(ta, tb, b_bf16):
    """A product with >= 512 tiles of 256 x 256 runs on the large-tile kernels;
    compared on a sample of rows against float64."""
    torch = _torch()
    mo = _mo()
    M, N, K = 5890, 5900, 333
    g = torch.Generator(device="cuda").manual_seed(11)
    A = torch.randn(*((K, M) if ta else (M, K)), generator=g, device="cuda")
    B = torch.randn(*((N, K) if tb else (K, N)), generator=g, device="cuda")
    if b_bf16:
        B = B.to(torch.bfloat16)
    C = torch.randn(M, N, generator=g, device="cuda")
    C0 = C.clone()
    mo.native.opt_gemm(ta, tb, M, N, K, 1.5, A.data_ptr(), 0, A.shape[1], B.data_ptr(), b_bf16, B.shape[1],
                       -0.5, C.data_ptr(), N, mo.stream_ptr())
    torch.cuda.synchronize()
    rows = torch.tensor(sorted(set([0, 1, 255, 256, 257, M - 1] + list(range(3, M, 97)))), device="cuda")
    opA = (A.T if ta else A).double()[rows]
    opB = (B.T if tb else B).double()
    ref = 1.5 * (opA @ opB) - 0.5 * C0.double()[rows]
    bound = 2 * K * 2.0 ** -23 * (1.5 * (opA.abs() @ opB.abs()) + 0.5 * C0.double()[rows].abs())
    assert float(((C.double()[rows] - ref).abs() / bound).max()) <= 1.0
