"""GPU parity of the orthogonalised-momentum step (OPT_FLAG_MUON) against
oracle/muon.py, teacher-forced: each step the device's M_{t-1}, W_{t-1} and G
feed the oracle; gate M checks the momentum, gate MU the Newton-Schulz
result and the update (tests/contract.py)."""

import numpy as np
import pytest

import workloads
from tests import contract, harness

pytestmark = pytest.mark.gpu


def _run(wl, steps, iters, check_mats, capacity=None, fp32_mfma=False):
    import torch
    import matrix_optimizer_step_02_amd as mo
    hp = mo.Hyper(wl.beta1, wl.beta2, wl.eps, wl.lr, wl.K, wl.power_iters, capacity or wl.capacity_bytes,
                  muon=True, ns_iters=iters, fp32_mfma=fp32_mfma)
    states = [mo.new_state(s.m, s.n, wl.m_dtype, "cuda", W0=workloads.initial_weight(wl, i, "cuda"), bases=False)
              for i, s in enumerate(wl.matrices)]
    grp = mo.RotatedAdamGroup(states, hp)
    ohp = harness.oracle_hyper(wl)
    failures = []
    for t in range(1, steps + 1):
        harness.load_gradients(wl, states, t)
        torch.cuda.synchronize()
        keys = ("W", "G", "M")
        before = {i: harness.snap(states[i], keys) for i in check_mats}
        grp.step()
        torch.cuda.synchronize()
        for i in check_mats:
            a, b = before[i], harness.snap(states[i], keys)
            reps = [contract.gate_momentum(a["M"], a["G"], b["M"], wl.beta1, wl.m_dtype),
                    contract.gate_muon(a["W"], b["M"], b["W"], ohp, iters)]
            line = f"t={t} mat={i} {wl.matrices[i].m}x{wl.matrices[i].n}: " + "; ".join(map(str, reps))
            print(line, flush=True)
            failures += [line for r in reps if not r.ok]
    grp.close()
    assert not failures, "\n".join(failures)


@pytest.mark.parametrize("m_dtype,iters,fp32_mfma", [("f32", 1, False), ("bf16", 5, False), ("f32", 10, False),
                                                     ("bf16", 5, True)])
def test_muon_ragged_shapes(m_dtype, iters, fp32_mfma):
    """Ragged shapes; the Newton-Schulz products on bf16 MFMAs (the default)
    and on fp32 MFMAs."""
    mats = (workloads.MatrixSpec("a", 37, 53), workloads.MatrixSpec("b", 130, 67),
            workloads.MatrixSpec("c", 200, 200), workloads.MatrixSpec("d", 64, 96))
    wl = workloads.Workload("ragged_mu", 7, "ragged", mats, m_dtype, K=0, power_iters=1, steps=3,
                            grad_kind="iid", grad_std=1e-2)
    _run(wl, 3, iters, range(len(mats)), fp32_mfma=fp32_mfma)


def test_muon_layer_shapes_several_micro_groups():
    """The layer workload (1024 x 3072 wide, 3072 x 1024 tall, 1024^2) in
    several 16 MiB micro-groups sharing one scratch."""
    wl = workloads.get("layer")
    _run(wl, 3, 5, [0, 4, 6], capacity=1 << 24)


def test_muon_rejects_the_basis_entry_points():
    import matrix_optimizer_step_02_amd as mo
    st = [mo.new_state(16, 24, "f32", "cuda", bases=False)]
    grp = mo.RotatedAdamGroup(st, mo.Hyper(muon=True, ns_iters=3))
    for fn in (lambda: grp.refresh_basis(1), lambda: grp.health(), lambda: grp.reorthonormalize(1)):
        with pytest.raises(mo.native.MatoptError) as e:
            fn()
        assert e.value.status == mo.native.OPT_EUNSUPPORTED
    grp.close()


@pytest.mark.timeout(900)
def test_muon_qwen3_1p7b_full_size_sampled():
    """The Qwen3-1.7B-shaped set in the bench's configuration (5 iterations),
    gated on the first and last layer's q, k, up and down."""
    wl = workloads.get("qwen3_1p7b")
    idx = [i for i, s in enumerate(wl.matrices)
           if s.layer in (0, 27) and s.name.split(".")[1] in ("q", "k", "up", "down")]
    _run(wl, 2, 5, idx)
