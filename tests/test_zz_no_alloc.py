"""The QR entry point that allocates nothing (opt_orthonormalize_static),
against the workspace entry point it shares its kernels with."""

import numpy as np
import pytest

pytestmark = pytest.mark.gpu


def _call(static, Z, ws=None):
    import torch
    import matrix_optimizer_step_02_amd as mo
    N = mo.native
    d = Z.shape[0]
    Zd = torch.tensor(Z, dtype=torch.float32, device="cuda").contiguous()
    Q = torch.full_like(Zd, float("nan"))
    if static:
        N.opt_orthonormalize_static(Zd.data_ptr(), Q.data_ptr(), d, mo.stream_ptr())
    else:
        nb = N.opt_orthonormalize_workspace_size(d)
        ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
        N.opt_orthonormalize(Zd.data_ptr(), Q.data_ptr(), d, ws.data_ptr(), nb, mo.stream_ptr())
    torch.cuda.synchronize()
    return Q.double().cpu().numpy(), Zd.double().cpu().numpy()


def test_static_entry_point_equals_the_workspace_one_on_two_calls():
    """Two calls in a row, the second with a smaller input, so that the
    second runs on what the first left in the fixed scratch: each result is
    bitwise the workspace entry point's (same kernels, same order), and
    within the fp32 bound of the oracle's positive-diagonal factor."""
    import oracle
    for d, seed in ((1000, 1), (300, 2)):
        print(f"static qr d={d}", flush=True)
        rng = np.random.default_rng(seed)
        Z = oracle.round_f32(np.eye(d) + 0.3 * rng.standard_normal((d, d)) / np.sqrt(d))
        Qs, Zs = _call(True, Z)
        Qw, Zw = _call(False, Z)
        assert np.array_equal(Qs, Qw) and np.array_equal(Zs, Zw)
        assert np.max(np.abs(Qs - oracle.orthonormal_factor(Z))) < 2e-5
        assert np.max(np.abs(Qs.T @ Qs - np.eye(d))) < 1e-5


def test_static_entry_point_rejects_orders_past_its_scratch():
    import matrix_optimizer_step_02_amd as mo
    N = mo.native
    with pytest.raises(N.MatoptError) as e:
        N.opt_orthonormalize_static(1 << 40, 1 << 41, N.OPT_STATIC_MAX_DIM + 1, 0)
    assert e.value.status == N.OPT_EUNSUPPORTED
    with pytest.raises(N.MatoptError) as e:
        N.opt_orthonormalize_static(1 << 40, 1 << 41, 0, 0)
    assert e.value.status == N.OPT_EINVAL
