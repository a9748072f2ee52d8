"""Writes tests/golden/tiny_trajectory.json from the oracle alone.

The pages print no worked example, so this fixture is a regression record of
the oracle on the 4 x (64x128) workload (CPU draws from the workloads module):
it pins the oracle against later unintended changes of its arithmetic. Run
``python -m tests.golden.make_golden`` from the repository root to rewrite it.
"""

import json
import os

import numpy as np


def tiny_trajectory():
    import oracle
    import workloads
    wl = workloads.get("tiny")
    hp = oracle.Hyper(wl.beta1, wl.beta2, wl.eps, wl.lr, wl.K, wl.power_iters)
    out = {}
    for i in range(2):
        st = oracle.OracleState.fresh(workloads.initial_weight(wl, i).double().numpy(), wl.m_dtype)
        for t in range(1, wl.steps + 1):
            G = workloads.gradient(wl, i, t).double().numpy()
            oracle.step(st, G, hp)
            out[f"m{i}.t{t}.W[0,:6]"] = st.W[0, :6].tolist()
            out[f"m{i}.t{t}.v[:3,0]"] = st.v[:3, 0].tolist()
            out[f"m{i}.t{t}.U[:3,0]"] = st.U[:3, 0].tolist()
            out[f"m{i}.t{t}.V[:3,1]"] = st.V[:3, 1].tolist()
            out[f"m{i}.t{t}.normW"] = [float(np.linalg.norm(st.W))]
    return out


if __name__ == "__main__":
    path = os.path.join(os.path.dirname(__file__), "tiny_trajectory.json")
    with open(path, "w") as f:
        json.dump(tiny_trajectory(), f, indent=1, sort_keys=True)
    print("wrote", path)
