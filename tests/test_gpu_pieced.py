"""GPU parity of the fp32 products on bf16 MFMAs.

By default the library runs the fp32 products of the rotations and of the
refresh on bf16 MFMAs at fp32 accuracy: each fp32 operand splits exactly into
three bf16 pieces and the six piece products that matter accumulate in fp32
(the terms left out are below 2^-23 of each product); a bf16 momentum (sides
multiples of 8) is exactly bf16, so the larger product of its chain (U^T M
when m > n, M V otherwise) runs as three bf16 products against stored pieces
of the basis. The step must pass gates M, A and B at the fp32 tolerance
(tau = 1e-4, not the 2e-2 of a bf16 M), as the all-fp32 path
(OPT_FLAG_FP32_MFMA) does on the same inputs.
"""

import numpy as np
import pytest

import oracle
import workloads
from tests import contract, harness

pytestmark = pytest.mark.gpu

# tall (U^T M pieced, K = m), wide and square (M V pieced, K = n); K values
# that are not multiples of the 64-deep slab; one matrix with a side that is
# not a multiple of 8 (all-fp32 in the same grouped launches)
SHAPES = ((200, 72), (72, 264), (136, 136), (64, 64), (520, 24), (24, 520), (130, 67))


def _hyper(wl, fp32_only):
    import matrix_optimizer_step_02_amd as mo
    return mo.Hyper(wl.beta1, wl.beta2, wl.eps, wl.lr, wl.K, wl.power_iters, wl.capacity_bytes,
                    fp32_mfma=fp32_only)


def _workload(K, steps, capacity, m_dtype="bf16"):
    mats = tuple(workloads.MatrixSpec(f"p{i}", m, n) for i, (m, n) in enumerate(SHAPES))
    return workloads.Workload("pieced", 13, "pieced", mats, m_dtype, K=K, power_iters=1, steps=steps,
                              grad_kind="iid", grad_std=1e-2, capacity_bytes=capacity)


@pytest.mark.parametrize("fp32_only,m_dtype", [(False, "bf16"), (True, "bf16"), (False, "f32")])
def test_pieced_step_fp32_tolerance(fp32_only, m_dtype):
    """Refresh at t = 1 and 3, three micro-groups: gates M, A and B with the
    fp32 tolerance on every matrix and step, for the default (bf16-piece)
    products and the all-fp32 ones."""
    import torch
    wl = _workload(K=2, steps=3, capacity=200 * 1024, m_dtype=m_dtype)
    grp, states = harness.build_group(wl, hp=_hyper(wl, fp32_only))
    hp = harness.oracle_hyper(wl)
    failures = []
    for t in range(1, 4):
        harness.load_gradients(wl, states, t)
        torch.cuda.synchronize()
        before = [harness.snap(s) for s in states]
        grp.step()
        torch.cuda.synchronize()
        for i, st in enumerate(states):
            a, b = before[i], harness.snap(st)
            reps = [contract.gate_momentum(a["M"], a["G"], b["M"], wl.beta1, wl.m_dtype)]
            if oracle.refresh_due(t, wl.K):
                reps += contract.gate_refresh(b["M"], a["U"], a["V"], b["U"], b["V"], wl.power_iters)
            # the fp32 tolerance although M is bf16: the oracle consumes the device's M
            reps += contract.gate_apply(a["W"], a["v"], b["M"], a["G"], b["U"], b["V"], b["W"], b["v"], hp,
                                        "f32")
            line = f"fp32_only={fp32_only} {m_dtype} t={t} mat={i} {SHAPES[i]}: " + "; ".join(map(str, reps))
            print(line, flush=True)
            failures += [line for r in reps if not r.ok]
    grp.close()
    assert not failures, "\n".join(failures)


def _dense_bases(wl, seed=5):
    import torch
    rng = np.random.default_rng(seed)
    bases = []
    for s in wl.matrices:
        pair = []
        for d in (s.m, s.n):
            q, r = np.linalg.qr(rng.standard_normal((d, d)))
            pair.append(torch.tensor(q * np.sign(np.diag(r)), dtype=torch.float32))
        bases.append(pair)
    return bases


def _run_dense(wl, hp_dev, bases, gate=True):
    """Three steps from the given bases (K = 0); every step gated against the
    oracle at the fp32 tolerance (teacher-forced). Returns the final W, v, M
    and the initial W of every matrix."""
    import torch
    grp, states = harness.build_group(wl, hp=hp_dev)
    for st, (U, V) in zip(states, bases):
        st["U"].copy_(U)
        st["V"].copy_(V)
    grp.t = 0   # set_step: the copies of the bases follow the new U, V
    W0 = [st["W"].double().cpu().numpy() for st in states]
    hp = harness.oracle_hyper(wl)
    failures = []
    for t in range(1, 4):
        harness.load_gradients(wl, states, t)
        torch.cuda.synchronize()
        before = [harness.snap(s) for s in states] if gate else None
        grp.step()
        torch.cuda.synchronize()
        for i, st in enumerate(states if gate else []):
            a, b = before[i], harness.snap(st)
            reps = contract.gate_apply(a["W"], a["v"], b["M"], a["G"], b["U"], b["V"], b["W"], b["v"], hp, "f32")
            line = f"dense t={t} mat={i} {SHAPES[i]}: " + "; ".join(map(str, reps))
            print(line, flush=True)
            failures += [line for r in reps if not r.ok]
    out = [harness.snap(st, ("W", "v", "M")) for st in states]
    grp.close()
    assert not failures, "\n".join(failures)
    return out, W0


@pytest.mark.parametrize("fp32_only", [False, True])
def test_dense_bases_fp32_tolerance(fp32_only):
    """Fixed random orthogonal bases (K = 0): G~ = U^T G V is dense, so u is
    well conditioned nearly everywhere; gate B at the fp32 tolerance at every
    step. (The two paths agree with each other only as two fp32-accurate
    results do: where G~ is tiny, u = m~ / sqrt(v) turns the rounding of G~
    into larger relative changes, which gate B's error model accounts for.)"""
    wl = _workload(K=0, steps=3, capacity=1 << 29)
    _run_dense(wl, _hyper(wl, fp32_only), _dense_bases(wl))
