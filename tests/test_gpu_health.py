"""GPU parity of the state checks (opt_group_health) and of the basis
re-orthonormalisation (opt_group_reorthonormalize) against oracle/health.py.

Bounds: v statistics are float64 sums of the same fp32 values (relative
1e-9); the drift is read from an fp32 Gram matrix, whose entries carry a
rounding error of a few 1e-7 for an orthonormal basis, so device and oracle
drifts agree to 2e-6 absolute plus 1e-3 relative; Newton-Schulz steps reach
the polar factor up to fp32 rounding (2e-6 per entry at these orders).
"""

import numpy as np
import pytest

import workloads
from oracle import health as H
from tests import harness

pytestmark = pytest.mark.gpu


def _perturb_bases(states, scale, seed):
    """U, V <- orthogonal + scale * noise (drift ~ scale)."""
    import torch
    rng = np.random.default_rng(seed)
    for st in states:
        for key in ("U", "V"):
            d = st[key].shape[0]
            Q, R = np.linalg.qr(rng.standard_normal((d, d)))
            X = Q * np.sign(np.diag(R)) + scale * rng.standard_normal((d, d)) / np.sqrt(d)
            st[key].copy_(torch.tensor(X, dtype=torch.float32))


def _check_health(grp, states, drift_abs=2e-6):
    rep = grp.health()
    for i, st in enumerate(states):
        s = harness.snap(st)
        m_abs, std, vmin, vmax = H.v_stats(s["v"])
        r = rep[i]
        print(f"mat {i} {s['W'].shape}: orth_U {r['orth_U']:.3e} (oracle {H.orth_drift(s['U']):.3e}) "
              f"orth_V {r['orth_V']:.3e} v_mean_abs {r['v_mean_abs']:.4e} std {r['v_std']:.4e}", flush=True)
        for key, dev in (("U", r["orth_U"]), ("V", r["orth_V"])):
            ref = H.orth_drift(s[key])
            assert abs(dev - ref) <= drift_abs + 1e-3 * ref, (i, key, dev, ref)
        if np.all(np.isfinite(s["v"])):
            assert r["v_mean_abs"] == pytest.approx(m_abs, rel=1e-9, abs=1e-300)
            assert r["v_std"] == pytest.approx(std, rel=1e-6, abs=1e-12 * max(m_abs, 1e-30))
        else:
            assert not np.isfinite(r["v_mean_abs"]) and not np.isfinite(m_abs)
        assert r["v_min"] == vmin and r["v_max"] == vmax
        assert r["nonfinite"] == H.nonfinite(s["W"], s["M"], s["v"])
    return rep


def test_health_after_steps_matches_oracle():
    wl = workloads.get("layer")
    grp, states = harness.build_group(wl)
    for t in range(1, 4):
        harness.load_gradients(wl, states, t)
        grp.step()
    rep = _check_health(grp, states)
    assert all(r["orth_U"] < 1e-5 and r["orth_V"] < 1e-5 for r in rep)
    grp.close()


@pytest.mark.parametrize("m_dtype", ["f32", "bf16"])
def test_reorthonormalize_reaches_polar_factor_ragged_shapes_several_batches(m_dtype):
    """Odd orders (unaligned, non-vector loads), m < n and m > n, and a refresh
    cap small enough to split the matrices over several refresh batches."""
    import torch
    import matrix_optimizer_step_02_amd as mo
    mats = (workloads.MatrixSpec("a", 37, 53), workloads.MatrixSpec("b", 130, 67),
            workloads.MatrixSpec("c", 1, 9), workloads.MatrixSpec("d", 300, 300),
            workloads.MatrixSpec("e", 1100, 260))
    wl = workloads.Workload("ragged", 7, "ragged", mats, m_dtype, K=1, power_iters=1, steps=2,
                            grad_kind="iid", grad_std=1e-2)
    hp = mo.Hyper(wl.beta1, wl.beta2, wl.eps, wl.lr, 0, 1, refresh_capacity_bytes=8 << 20)
    grp, states = harness.build_group(wl, hp=hp)
    harness.load_gradients(wl, states, 1)
    grp.step()
    _perturb_bases(states, 1e-3, 5)
    torch.cuda.synchronize()
    before = [harness.snap(st, ("U", "V")) for st in states]
    _check_health(grp, states)
    grp.reorthonormalize(2)
    torch.cuda.synchronize()
    for i, st in enumerate(states):
        after = harness.snap(st, ("U", "V"))
        for key in ("U", "V"):
            ref = H.polar_factor(before[i][key])
            err = np.max(np.abs(after[key] - ref))
            print(f"mat {i} {key} {ref.shape}: |X - polar| {err:.2e} drift {H.orth_drift(after[key]):.2e}", flush=True)
            assert err <= 2e-6
            assert H.orth_drift(after[key]) <= 2e-6
    _check_health(grp, states)
    grp.close()


def test_health_counts_nonfinite_and_extremes():
    import torch
    wl = workloads.get("tiny")
    grp, states = harness.build_group(wl)
    harness.load_gradients(wl, states, 1)
    grp.step()
    states[0]["W"][3, 5] = float("nan")
    states[1]["v"][0, 0] = float("inf")
    states[2]["M"][7, 1] = float("-inf")
    states[3]["v"][2, 2] = -1.0
    torch.cuda.synchronize()
    rep = _check_health(grp, states)
    assert [r["nonfinite"] for r in rep] == [1, 1, 1, 0]
    assert rep[3]["v_min"] == -1.0
    grp.close()


def test_reorthonormalize_zero_iterations_is_a_no_op_and_orthogonal_bases_stay():
    import torch
    wl = workloads.get("tiny")
    grp, states = harness.build_group(wl)
    for t in range(1, 3):
        harness.load_gradients(wl, states, t)
        grp.step()
    torch.cuda.synchronize()
    before = [harness.snap(st, ("U", "V")) for st in states]
    grp.reorthonormalize(0)
    torch.cuda.synchronize()
    for i, st in enumerate(states):
        after = harness.snap(st, ("U", "V"))
        assert np.array_equal(after["U"], before[i]["U"]) and np.array_equal(after["V"], before[i]["V"])
    grp.reorthonormalize(1)
    torch.cuda.synchronize()
    for i, st in enumerate(states):
        after = harness.snap(st, ("U", "V"))
        for key in ("U", "V"):
            assert np.max(np.abs(after[key] - before[i][key])) <= 2e-6
    grp.close()
