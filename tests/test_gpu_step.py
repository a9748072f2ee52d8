"""GPU parity of the whole step against the oracle (teacher-forced gates).

Every gate consumes the device's own persisted state of the previous phase;
the gates and their tolerances are described in tests/contract.py.
"""

import numpy as np
import pytest

import oracle
import workloads
from tests import contract, harness, textbook

pytestmark = pytest.mark.gpu


def _run_gated(wl, steps, check_steps, check_mats, forward_max_d=1100):
    import torch
    grp, states = harness.build_group(wl)
    hp = harness.oracle_hyper(wl)
    failures = []
    for t in range(1, steps + 1):
        harness.load_gradients(wl, states, t)
        torch.cuda.synchronize()
        check = t in check_steps
        before = {i: harness.snap(states[i]) for i in check_mats} if check else {}
        grp.step()
        torch.cuda.synchronize()
        assert grp.t == t
        if not check:
            continue
        refreshed = oracle.refresh_due(t, wl.K)
        for i in check_mats:
            a, b = before[i], harness.snap(states[i])
            reps = [contract.gate_momentum(a["M"], a["G"], b["M"], wl.beta1, wl.m_dtype)]
            if refreshed:
                reps += contract.gate_refresh(b["M"], a["U"], a["V"], b["U"], b["V"], wl.power_iters,
                                              forward_max_d)
            else:
                same = np.array_equal(a["U"], b["U"]) and np.array_equal(a["V"], b["V"])
                reps.append(contract.GateReport("A.unchanged", same))
            reps += contract.gate_apply(a["W"], a["v"], b["M"], a["G"], b["U"], b["V"], b["W"], b["v"],
                                        hp, wl.m_dtype)
            line = f"t={t} mat={i} {wl.matrices[i].m}x{wl.matrices[i].n}: " + "; ".join(map(str, reps))
            print(line, flush=True)
            failures += [line for r in reps if not r.ok]
    grp.close()
    assert not failures, "\n".join(failures)


def test_tiny_all_steps():
    wl = workloads.get("tiny")
    _run_gated(wl, wl.steps, set(range(1, wl.steps + 1)), range(len(wl.matrices)))


def test_ragged_shapes_refresh_every_step():
    """Shapes that are not multiples of any tile or panel size, m < n and m > n,
    fp32 and bf16 momentum, refreshed every step with 2 passes."""
    for m_dtype in ("f32", "bf16"):
        mats = (workloads.MatrixSpec("a", 37, 53), workloads.MatrixSpec("b", 130, 67),
                workloads.MatrixSpec("c", 1, 9), workloads.MatrixSpec("d", 200, 200))
        wl = workloads.Workload("ragged", 7, "ragged", mats, m_dtype, K=1, power_iters=2, steps=3,
                                grad_kind="iid", grad_std=1e-2)
        _run_gated(wl, 3, {1, 2, 3}, range(len(mats)))


def test_layer_sampled_steps():
    wl = workloads.get("layer")
    _run_gated(wl, 12, {1, 2, 10, 11, 12}, [0, 4, 6])


def test_layer_fp32_momentum_sampled_steps():
    wl = workloads.get("layer_f32m")
    _run_gated(wl, 11, {1, 11}, [1, 5])


def test_identity_bases_is_coordinatewise_adam():
    """K = 0 with U = I, V = I: the device step is coordinate-wise Adam; every
    rotation product multiplies by exact ones and zeros, so only the
    elementwise fp32 roundings differ from the float64 textbook path."""
    import torch
    import matrix_optimizer_step_02_amd as mo
    wl = workloads.get("tiny")
    hp = mo.Hyper(wl.beta1, wl.beta2, wl.eps, wl.lr, 0, 1)
    grp, states = harness.build_group(wl, hp=hp)
    ref = [harness.snap(s) for s in states]
    w = [r["W"] for r in ref]
    m = [np.zeros_like(x) for x in w]
    v = [np.zeros_like(x) for x in w]
    for t in range(1, 4):
        harness.load_gradients(wl, states, t)
        G = [harness.snap(s, ("G",))["G"] for s in states]
        grp.step()
        torch.cuda.synchronize()
        for i, s in enumerate(states):
            w[i], m[i], v[i] = textbook.adam_coordinatewise(w[i], m[i], v[i], G[i], wl.beta1, wl.beta2,
                                                            wl.eps, wl.lr, textbook.f32)
            b = harness.snap(s)
            assert np.array_equal(b["U"], np.eye(b["U"].shape[0]))
            assert contract.maxrel(b["M"], m[i]) <= 2 ** -23
            assert contract.maxrel(b["v"], v[i]) <= 2 ** -22
            assert np.max(np.abs(b["W"] - w[i])) <= 8 * 2 ** -24 * (np.max(np.abs(w[i])) + 10 * wl.lr)
    grp.close()


@pytest.mark.timeout(900)
def test_qwen3_1p7b_full_size_sampled():
    """The whole Qwen3-1.7B-shaped set (196 matrices, 11 micro-groups, the
    launch configuration the bench times); gates on the first and last layer's
    matrices of every shape, at the refresh step t = 1, the plain step t = 2
    and the last step of the epoch t = K = 10 (where v is established and the
    bound is tau alone). Bases of order > 1100 are compared with the oracle on
    their leading 256 columns."""
    wl = workloads.get("qwen3_1p7b")
    idx = [i for i, s in enumerate(wl.matrices) if s.layer in (0, 27) and s.name.split(".")[1] in ("q", "k", "up", "down")]
    _run_gated(wl, 10, {1, 2, 10}, idx)


@pytest.mark.timeout(900)
def test_microgroup_512mib_full_size_sampled():
    """One exactly-full 512 MiB micro-group of fp32 state with two power
    iterations per refresh (K = 5): the refresh steps t = 1 and t = 6 and the
    plain steps t = 2 and t = 5 (the epoch's last), on the largest matrix of
    each orientation and one of the small ones."""
    wl = workloads.get("microgroup_512mib")
    _run_gated(wl, 6, {1, 2, 5, 6}, [0, 2, 6])


@pytest.mark.timeout(900)
def test_qwen3_8b_half_full_size_sampled():
    """Layers 0-17 of the Qwen3-8B shapes at real size (126 matrices, bf16
    momentum, anisotropic gradients): gates at the refresh step t = 1 and the
    plain steps t = 2 and t = K = 5 on the first layer's q, k, down and the
    last layer's up."""
    wl = workloads.get("qwen3_8b_half")
    idx = [i for i, s in enumerate(wl.matrices)
           if (s.layer == 0 and s.name.split(".")[1] in ("q", "k", "down"))
           or (s.layer == 17 and s.name.split(".")[1] == "up")]
    assert len(idx) == 4
    _run_gated(wl, 5, {1, 2, 5}, idx)


def test_rotations_follow_bases_changed_between_steps():
    """The fp32 rotations read U^T from a workspace copy of U: after
    refresh_basis, and after the caller writes new orthogonal U, V and calls
    set_step, the next step must rotate with the new bases (gate B against
    the bases as they are before that step)."""
    import torch
    mats = (workloads.MatrixSpec("a", 37, 53), workloads.MatrixSpec("b", 130, 67),
            workloads.MatrixSpec("c", 96, 96))
    wl = workloads.Workload("bases_changed", 11, "bases changed", mats, "bf16", K=0, power_iters=1, steps=5,
                            grad_kind="iid", grad_std=1e-2)
    grp, states = harness.build_group(wl)
    hp = harness.oracle_hyper(wl)
    rng = np.random.default_rng(23)
    failures = []
    for t in range(1, 6):
        if t == 3:
            grp.refresh_basis(1)
        if t == 4:
            for st in states:
                for key in ("U", "V"):
                    d = st[key].shape[0]
                    q, r = np.linalg.qr(rng.standard_normal((d, d)))
                    st[key].copy_(torch.tensor(q * np.sign(np.diag(r)), dtype=torch.float32))
            grp.t = grp.t
        harness.load_gradients(wl, states, t)
        torch.cuda.synchronize()
        before = [harness.snap(s) for s in states]
        grp.step()
        torch.cuda.synchronize()
        for i, st in enumerate(states):
            a, b = before[i], harness.snap(st)
            assert np.array_equal(a["U"], b["U"]) and np.array_equal(a["V"], b["V"])
            reps = [contract.gate_momentum(a["M"], a["G"], b["M"], wl.beta1, wl.m_dtype)]
            reps += contract.gate_apply(a["W"], a["v"], b["M"], a["G"], b["U"], b["V"], b["W"], b["v"], hp,
                                        wl.m_dtype)
            line = f"t={t} mat={i}: " + "; ".join(map(str, reps))
            print(line, flush=True)
            failures += [line for r in reps if not r.ok]
    grp.close()
    assert not failures, "\n".join(failures)
