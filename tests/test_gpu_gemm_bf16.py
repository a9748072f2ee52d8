"""GPU tests of the bf16 GEMM building block (opt_gemm_bf16), through the C ABI.

C = alpha A B^T + beta C with A (M x K), B (N x K) bf16. A product of two
bf16 values is exact in binary32, so the device result differs from the
float64 product of the same bf16 inputs only by its binary32 accumulation:
|C - ref| <= 2 K 2^-23 (|alpha| |A| |B|^T + |beta C0|). A bf16 C is that
accumulation rounded to nearest even, so it must lie between the roundings of
ref minus and plus the bound (rounding is monotone).
"""

import numpy as np
import pytest

import oracle

pytestmark = pytest.mark.gpu


def _torch():
    import torch
    return torch


def _mo():
    import matrix_optimizer_step_02_amd as mo
    return mo


def _case(M, N, K, alpha=1.0, beta=0.0, c_bf16=False, lda=None, ldb=None, seed=0):
    torch = _torch()
    mo = _mo()
    g = torch.Generator(device="cuda").manual_seed(seed)
    lda = lda or max(K, 8)
    ldb = ldb or max(K, 8)
    # row strides past K hold values the product must not read
    A = torch.randn(M, lda, generator=g, device="cuda").to(torch.bfloat16)
    B = torch.randn(N, ldb, generator=g, device="cuda").to(torch.bfloat16)
    C = torch.randn(M, N, generator=g, device="cuda")
    if c_bf16:
        C = C.to(torch.bfloat16)
    C0 = C.double().cpu().numpy()
    mo.native.opt_gemm_bf16(M, N, K, alpha, A.data_ptr(), lda, B.data_ptr(), ldb, beta, C.data_ptr(),
                             int(c_bf16), N, mo.stream_ptr())
    torch.cuda.synchronize()
    An = A.double().cpu().numpy()[:, :K]
    Bn = B.double().cpu().numpy()[:, :K]
    ref = alpha * (An @ Bn.T) + beta * C0
    E = 2 * max(K, 1) * 2.0 ** -23 * (abs(alpha) * (np.abs(An) @ np.abs(Bn).T) + np.abs(beta * C0))
    got = C.double().cpu().numpy()
    if not c_bf16:
        return float(np.max(np.abs(got - ref) / (E + 1e-30))), 0
    lo = oracle.round_bf16(ref - E)
    hi = oracle.round_bf16(ref + E)
    outside = int(np.count_nonzero((got < lo) | (got > hi)))
    differ = int(np.count_nonzero(got != oracle.round_bf16(ref)))
    return outside, differ


SHAPES = [(130, 67, 40), (256, 384, 512), (1, 1, 8), (33, 129, 8), (200, 300, 1000), (600, 520, 136)]


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_fp32_out_ragged(M, N, K):
    print(f"gemm16 f32 {M}x{N}x{K}", flush=True)
    r, _ = _case(M, N, K, alpha=0.75, beta=0.5)
    assert r <= 1.0, r


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_bf16_out_ragged(M, N, K):
    print(f"gemm16 bf16 {M}x{N}x{K}", flush=True)
    outside, differ = _case(M, N, K, alpha=1.25, c_bf16=True)
    assert outside == 0
    assert differ <= max(2, M * N // 1000), differ


def test_strided_operands_skip_padding():
    print("gemm16 strided", flush=True)
    r, _ = _case(96, 80, 72, lda=136, ldb=88, alpha=1.0, beta=1.0)
    assert r <= 1.0, r


@pytest.mark.parametrize("M,N,K", [(4096, 4096, 512), (4100, 4000, 264)])
def test_large_tiles(M, N, K):
    """At least 256 tiles of 256 x 256: the large configuration, with a
    ragged edge and a partial last slab in the second case."""
    print(f"gemm16 large {M}x{N}x{K}", flush=True)
    r, _ = _case(M, N, K, alpha=-0.5, beta=1.0)
    assert r <= 1.0, r


def test_empty_k_scales_c():
    r, _ = _case(70, 90, 0, alpha=1.0, beta=2.0)
    assert r <= 1.0
