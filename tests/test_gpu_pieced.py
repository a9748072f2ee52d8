"""GPU parity of the pieced momentum rotation.

With fp32 rotations and a bf16 momentum whose sides are multiples of 8, the
library runs the larger product of M's chain (U^T M when m > n, M V
otherwise) as three bf16 MFMA products against the exact bf16 pieces
hi + mid + lo of the fp32 basis, accumulated in one fp32 chain. M is exactly
bf16, so the product equals the fp32 one up to accumulation order: the step
must pass gate B at the fp32 tolerance (tau = 1e-4), as the all-fp32 path
(OPT_FLAG_FP32_MOMENTUM_ROTATION) does on the same inputs, and the two paths
must agree where the update is well conditioned.
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
                    fp32_momentum_rotation=fp32_only)


def _workload(K, steps, capacity):
    mats = tuple(workloads.MatrixSpec(f"p{i}", m, n) for i, (m, n) in enumerate(SHAPES))
    return workloads.Workload("pieced", 13, "pieced", mats, "bf16", K=K, power_iters=1, steps=steps,
                              grad_kind="iid", grad_std=1e-2, capacity_bytes=capacity)


@pytest.mark.parametrize("fp32_only", [False, True])
def test_pieced_step_fp32_tolerance(fp32_only):
    """Refresh at t = 1 and 3, three micro-groups: gates M, A and B with the
    fp32 tolerance on every matrix and step."""
    import torch
    wl = _workload(K=2, steps=3, capacity=200 * 1024)
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
            line = f"fp32_only={fp32_only} t={t} mat={i} {SHAPES[i]}: " + "; ".join(map(str, reps))
            print(line, flush=True)
            failures += [line for r in reps if not r.ok]
    grp.close()
    assert not failures, "\n".join(failures)


def test_pieced_matches_fp32_products_with_dense_bases():
    """Fixed random orthogonal bases (K = 0): G~ = U^T G V is dense, so u is
    well conditioned everywhere and the pieced and all-fp32 paths must give
    the same v and W up to fp32 rounding, step after step."""
    import torch
    wl = _workload(K=0, steps=3, capacity=1 << 29)
    rng = np.random.default_rng(5)
    bases = []
    for s in wl.matrices:
        pair = []
        for d in (s.m, s.n):
            q, r = np.linalg.qr(rng.standard_normal((d, d)))
            pair.append(torch.tensor(q * np.sign(np.diag(r)), dtype=torch.float32))
        bases.append(pair)
    runs = []
    for fp32_only in (False, True):
        grp, states = harness.build_group(wl, hp=_hyper(wl, fp32_only))
        for st, (U, V) in zip(states, bases):
            st["U"].copy_(U)
            st["V"].copy_(V)
        grp.t = 0   # set_step: the copies of the bases follow the new U, V
        W0 = [st["W"].clone() for st in states]
        for t in range(1, 4):
            harness.load_gradients(wl, states, t)
            grp.step()
        torch.cuda.synchronize()
        runs.append([(harness.snap(st, ("W", "v", "M")), w0.double().cpu().numpy())
                     for st, w0 in zip(states, W0)])
        grp.close()
    bad = []
    for i, ((a, w0), (b, _)) in enumerate(zip(*runs)):
        assert np.array_equal(a["M"], b["M"]), f"mat {i}: M differs"
        dv = np.max(np.abs(a["v"] - b["v"])) / np.max(np.abs(b["v"]))
        dW = np.max(np.abs((a["W"] - w0) - (b["W"] - w0))) / np.max(np.abs(b["W"] - w0))
        print(f"mat {i} {SHAPES[i]}: v maxrel {dv:.2e}, dW maxrel {dW:.2e}", flush=True)
        if not (dv <= 1e-5 and dW <= 1e-4):
            bad.append((i, dv, dW))
    assert not bad, bad
