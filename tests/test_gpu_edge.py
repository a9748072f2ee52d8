"""GPU edge cases of the step: the largest supported order, a zero gradient
(the refresh then factorises a zero matrix), and a non-finite gradient, which
must stay inside its own matrix. Teacher-forced gates as in test_gpu_step."""

import numpy as np
import pytest

import oracle
import workloads
from tests import contract, harness

pytestmark = pytest.mark.gpu


def _gates(wl, i, a, b, hp, refreshed, sampled_bases=False):
    reps = [contract.gate_momentum(a["M"], a["G"], b["M"], wl.beta1, wl.m_dtype)]
    if refreshed:
        m, n = wl.matrices[i].m, wl.matrices[i].n
        for side, X0, X1, d in (("U", a["U"], b["U"], m), ("V", a["V"], b["V"], n)):
            if sampled_bases and d > 1100:
                reps.append(contract.gate_basis_sampled(X1, b["M"], X0, side, wl.power_iters, "A." + side))
            else:
                A = b["M"] @ b["M"].T if side == "U" else b["M"].T @ b["M"]
                reps.append(contract.gate_basis(X1, A, X0, min(m, n), wl.power_iters, "A." + side,
                                                ref32=lambda s=side, X=X0: contract.fp32_refresh(b["M"], X, s,
                                                                                               wl.power_iters)))
    reps += contract.gate_apply(a["W"], a["v"], b["M"], a["G"], b["U"], b["V"], b["W"], b["v"], hp, wl.m_dtype)
    return reps


@pytest.mark.timeout(900)
def test_largest_order_tall_and_wide():
    """16384 x 64 and 64 x 16384 (OPT_MAX_DIM rows, then columns): the
    16384-order refresh runs every block of the factorisation; its basis is
    checked on sampled rows and columns, the rest in full; two refresh steps."""
    import torch
    mats = (workloads.MatrixSpec("tall", 16384, 64), workloads.MatrixSpec("wide", 64, 16384))
    wl = workloads.Workload("maxdim", 8, "max order", mats, "f32", K=1, power_iters=1, steps=2,
                            grad_kind="iid", grad_std=1e-2)
    grp, states = harness.build_group(wl)
    hp = harness.oracle_hyper(wl)
    failures = []
    for t in (1, 2):
        harness.load_gradients(wl, states, t)
        torch.cuda.synchronize()
        before = [harness.snap(s) for s in states]
        print(f"maxdim step {t}", flush=True)
        grp.step()
        torch.cuda.synchronize()
        for i in range(2):
            reps = _gates(wl, i, before[i], harness.snap(states[i]), hp, True, sampled_bases=True)
            line = f"t={t} mat={i}: " + "; ".join(map(str, reps))
            print(line, flush=True)
            failures += [line for r in reps if not r.ok]
    grp.close()
    assert not failures, "\n".join(failures)


def _small_set():
    mats = (workloads.MatrixSpec("a", 48, 80), workloads.MatrixSpec("b", 96, 96), workloads.MatrixSpec("c", 70, 33))
    return workloads.Workload("edge", 9, "edge", mats, "f32", K=2, power_iters=1, steps=3, grad_kind="iid",
                              grad_std=1e-2)


def test_zero_gradient_first_step():
    """G = 0 at t = 1: M stays 0, the refresh factorises zero matrices (the
    positive-diagonal convention keeps the identity bases), v stays 0, u is 0
    and W does not move; a normal step follows."""
    import torch
    wl = _small_set()
    grp, states = harness.build_group(wl)
    hp = harness.oracle_hyper(wl)
    failures = []
    for t in (1, 2):
        harness.load_gradients(wl, states, t)
        if t == 1:
            for s in states:
                s["G"].zero_()
        torch.cuda.synchronize()
        before = [harness.snap(s) for s in states]
        grp.step()
        torch.cuda.synchronize()
        for i, s in enumerate(states):
            b = harness.snap(s)
            if t == 1:
                assert np.array_equal(b["W"], before[i]["W"]) and not b["M"].any() and not b["v"].any()
                assert np.array_equal(b["U"], np.eye(b["U"].shape[0])) and np.array_equal(b["V"], np.eye(b["V"].shape[0]))
            reps = _gates(wl, i, before[i], b, hp, oracle.refresh_due(t, wl.K))
            failures += [f"t={t} mat={i}: {r}" for r in reps if not r.ok]
    grp.close()
    assert not failures, "\n".join(failures)


def test_nonfinite_gradient_stays_in_its_matrix():
    """A NaN in one matrix's gradient propagates through that matrix's
    momentum, refresh and update (IEEE semantics, no error), and the other
    matrices of the same grouped launches step exactly as without it."""
    import torch
    wl = _small_set()
    grp, states = harness.build_group(wl)
    hp = harness.oracle_hyper(wl)
    harness.load_gradients(wl, states, 1)
    states[1]["G"][5, 7] = float("nan")
    torch.cuda.synchronize()
    before = [harness.snap(s) for s in states]
    grp.step()
    torch.cuda.synchronize()
    after = [harness.snap(s) for s in states]
    assert np.isnan(after[1]["M"][5, 7]) and np.isnan(after[1]["W"]).any()
    for i in (0, 2):
        reps = _gates(wl, i, before[i], after[i], hp, True)
        assert all(r.ok for r in reps), [str(r) for r in reps]
        assert np.isfinite(after[i]["W"]).all()
    h = grp.health()
    assert h[1]["nonfinite"] > 0 and h[0]["nonfinite"] == 0 and h[2]["nonfinite"] == 0
    grp.close()
