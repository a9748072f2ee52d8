"""GPU parity of the bases stored in 16 bits (OPT_FLAG_BF16_BASES with the
bf16 rotations) against oracle/bf16_rotation.py's storage mode,
teacher-forced (tests/contract.py): the refresh from the device's stored
bf16 bases, stored rounded (gate A16), and every step, the first included,
rotating with the stored bases (gate B16)."""

import numpy as np
import pytest

import oracle
import workloads
from tests import contract, harness

pytestmark = pytest.mark.gpu


def _run(wl, steps, check_steps, check_mats):
    import torch
    import matrix_optimizer_step_02_amd as mo
    hp_d = mo.Hyper(wl.beta1, wl.beta2, wl.eps, wl.lr, wl.K, wl.power_iters, wl.capacity_bytes,
                    bf16_rotation=True, bf16_bases=True)
    grp, states = harness.build_group(wl, "cuda", hp_d)
    assert states[0]["U"].dtype == torch.bfloat16
    hp = harness.oracle_hyper(wl)
    failures = []
    for t in range(1, steps + 1):
        harness.load_gradients(wl, states, t)
        torch.cuda.synchronize()
        check = t in check_steps
        before = {i: harness.snap(states[i]) for i in check_mats} if check else {}
        grp.step()
        torch.cuda.synchronize()
        if not check:
            continue
        refreshed = oracle.refresh_due(t, wl.K)
        for i in check_mats:
            a, b = before[i], harness.snap(states[i])
            reps = [contract.gate_momentum(a["M"], a["G"], b["M"], wl.beta1, wl.m_dtype)]
            if refreshed:
                reps += [contract.gate_basis16(b["U"], b["M"], a["U"], "U", wl.power_iters, "A16.U"),
                         contract.gate_basis16(b["V"], b["M"], a["V"], "V", wl.power_iters, "A16.V")]
            else:
                reps.append(contract.GateReport("A.unchanged", np.array_equal(a["U"], b["U"])
                                                and np.array_equal(a["V"], b["V"])))
            reps += contract.gate_apply_bf16(a["W"], a["v"], b["M"], a["G"], b["U"], b["V"], b["W"], b["v"], hp)
            line = f"t={t} mat={i} {wl.matrices[i].m}x{wl.matrices[i].n}: " + "; ".join(map(str, reps))
            print(line, flush=True)
            failures += [line for r in reps if not r.ok]
    grp.close()
    assert not failures, "\n".join(failures)


@pytest.mark.parametrize("m_dtype", ["f32", "bf16"])
def test_bf16_storage_ragged_shapes(m_dtype):
    """Orders that are and are not multiples of 8 (the caller's U serves as
    the rotations' copy only for the former), m < n and m > n, refreshed
    every step with two passes."""
    mats = (workloads.MatrixSpec("a", 37, 53), workloads.MatrixSpec("b", 130, 67),
            workloads.MatrixSpec("c", 64, 128), workloads.MatrixSpec("d", 200, 200))
    wl = workloads.Workload("ragged16", 8, "ragged, bases in 16 bits", mats, m_dtype, K=1, power_iters=2, steps=3,
                            grad_kind="iid", grad_std=1e-2)
    _run(wl, 3, {1, 2, 3}, range(len(mats)))


def test_bf16_storage_layer_sampled_steps():
    wl = workloads.get("layer")
    _run(wl, 12, {1, 2, 10, 11, 12}, [0, 4, 6])


def test_bf16_storage_rejects_fp32_bases_and_unsupported_calls():
    import torch
    import matrix_optimizer_step_02_amd as mo
    hp = mo.Hyper(bf16_rotation=True, bf16_bases=True)
    st = mo.new_state(16, 24, "bf16", "cuda")
    with pytest.raises(ValueError):
        mo.RotatedAdamGroup([st], hp)                       # fp32 U, V
    st = mo.new_state(16, 24, "bf16", "cuda", bases16=True)
    grp = mo.RotatedAdamGroup([st], hp)
    with pytest.raises(mo.MatoptError):
        grp.health()
    with pytest.raises(mo.MatoptError):
        grp.reorthonormalize(1)
    grp.close()
