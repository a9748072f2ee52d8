"""Device-side helpers for the GPU tests: build a group for a workload, feed
gradients, snapshot the caller-owned state."""

from __future__ import annotations

import numpy as np

import workloads


def hyper_of(wl):
    import matrix_optimizer_step_02_amd as mo
    return mo.Hyper(wl.beta1, wl.beta2, wl.eps, wl.lr, wl.K, wl.power_iters, wl.capacity_bytes)


def oracle_hyper(wl):
    import oracle
    return oracle.Hyper(wl.beta1, wl.beta2, wl.eps, wl.lr, wl.K, wl.power_iters)


def build_group(wl, device="cuda", hp=None):
    import matrix_optimizer_step_02_amd as mo
    hp = hp or hyper_of(wl)
    states = []
    for i, s in enumerate(wl.matrices):
        W0 = workloads.initial_weight(wl, i, device)
        states.append(mo.new_state(s.m, s.n, wl.m_dtype, device, W0=W0, bases16=hp.bf16_bases))
    grp = mo.RotatedAdamGroup(states, hp)
    return grp, states


def load_gradients(wl, states, t, device="cuda"):
    for i, st in enumerate(states):
        st["G"].copy_(workloads.gradient(wl, i, t, device))


def snap(st, keys=("W", "G", "M", "v", "U", "V")):
    import torch
    return {k: st[k].to(torch.float64).cpu().numpy() for k in keys}
