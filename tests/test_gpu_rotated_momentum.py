"""GPU parity of the rotated-momentum variant (OPT_FLAG_ROTATED_MOMENTUM)
against oracle/rotated_momentum.py, with the teacher-forced gates of
tests/contract.py: every step the device's persisted state before the step
feeds the oracle, and the refresh, the carried m~, v and W are compared."""

import numpy as np
import pytest

import oracle
import workloads
from tests import contract, harness

pytestmark = pytest.mark.gpu


def _build(wl, **hp_kw):
    import matrix_optimizer_step_02_amd as mo
    hp = mo.Hyper(wl.beta1, wl.beta2, wl.eps, wl.lr, wl.K, wl.power_iters, wl.capacity_bytes,
                  rotated_momentum=True, **hp_kw)
    states = []
    for i, s in enumerate(wl.matrices):
        W0 = workloads.initial_weight(wl, i, "cuda")
        states.append(mo.new_state(s.m, s.n, wl.m_dtype, "cuda", W0=W0, rotated_momentum=True))
    return mo.RotatedAdamGroup(states, hp), states


def _run(wl, steps, check_mats, events=None):
    import torch
    grp, states = _build(wl)
    hp = harness.oracle_hyper(wl)
    keys = ("W", "G", "M", "v", "U", "V", "Mt")
    failures = []
    valid = False
    for t in range(1, steps + 1):
        if events and t in events:
            events[t](grp)
            valid = False
        harness.load_gradients(wl, states, t)
        torch.cuda.synchronize()
        before = {i: harness.snap(states[i], keys) for i in check_mats}
        grp.step()
        torch.cuda.synchronize()
        refreshed = oracle.refresh_due(t, wl.K)
        recompute = refreshed or not valid
        for i in check_mats:
            a, b = before[i], harness.snap(states[i], keys)
            reps = [contract.gate_momentum(a["M"], a["G"], b["M"], wl.beta1, wl.m_dtype)]
            if refreshed:
                reps += contract.gate_refresh(b["M"], a["U"], a["V"], b["U"], b["V"], wl.power_iters)
            else:
                reps.append(contract.GateReport("A.unchanged", np.array_equal(a["U"], b["U"])
                                                and np.array_equal(a["V"], b["V"])))
            reps += contract.gate_apply_rotated_momentum(a["W"], a["v"], a["Mt"], b["M"], a["G"], b["U"], b["V"],
                                                         b["W"], b["v"], b["Mt"], hp, recompute)
            line = f"t={t} mat={i} {wl.matrices[i].m}x{wl.matrices[i].n}: " + "; ".join(map(str, reps))
            print(line, flush=True)
            failures += [line for r in reps if not r.ok]
        valid = True
    grp.close()
    assert not failures, "\n".join(failures)


@pytest.mark.parametrize("m_dtype", ["f32", "bf16"])
def test_rotated_momentum_across_refreshes(m_dtype):
    """Refresh every 3 steps (t = 1, 4, 7): recomputed m~ at refreshes,
    carried m~ in between; ragged shapes, both momentum storages."""
    mats = (workloads.MatrixSpec("a", 37, 53), workloads.MatrixSpec("b", 130, 67),
            workloads.MatrixSpec("c", 200, 200))
    wl = workloads.Workload("ragged_rm", 7, "ragged", mats, m_dtype, K=3, power_iters=1, steps=8,
                            grad_kind="iid", grad_std=1e-2)
    _run(wl, 8, range(len(mats)))


def test_rotated_momentum_recomputes_after_external_basis_change():
    """refresh_basis and set_step between steps invalidate the carried m~:
    the next step must recompute it from M with the new bases."""
    wl = workloads.get("layer")
    wl = workloads.Workload(wl.key, wl.index, wl.title, wl.matrices, wl.m_dtype, K=0, power_iters=1, steps=6,
                            grad_kind=wl.grad_kind, grad_std=wl.grad_std)
    events = {3: lambda g: g.refresh_basis(1), 5: lambda g: setattr(g, "t", g.t)}
    _run(wl, 6, [0, 4, 6], events)


def test_rotated_momentum_matches_method_on_qwen3_layer_shapes():
    """The layer workload with its own refresh period (K = 10): 12 steps
    cover a carried epoch and the refresh at t = 11."""
    wl = workloads.get("layer")
    _run(wl, 12, [1, 5, 6])
