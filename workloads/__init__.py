"""Seeded synthetic workloads: matrix shapes, hyper-parameters and input draws.

This module holds no arithmetic of the optimizer step. It only says which
matrices exist, with which storage types and hyper-parameters, and draws the
initial weights and per-step gradients from seeded generators. The device path
(through the binding) and the CPU oracle (in tests) both consume what it draws:
the oracle always receives the exact binary32 arrays the device saw.

The shapes stand in for the pages' training workloads (Qwen3 models trained on
unnamed data, LLaMA-7B); no dataset or trained weight is involved.

Seeding: every tensor is drawn from its own generator seeded from the tuple
(workload index, matrix index, step, stream tag) through numpy's SeedSequence,
so any one matrix or step can be regenerated alone.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field, replace
from typing import List, Tuple

import numpy as np

_TAG_W0 = 1
_TAG_G = 2
_TAG_SCALE = 3
_TAG_SHAPES = 4


@dataclass(frozen=True)
class MatrixSpec:
    name: str
    m: int
    n: int
    layer: int = 0
    uid: int = -1   # position in the full workload; seeds follow it, so subsets draw the same tensors


@dataclass(frozen=True)
class Workload:
    key: str
    index: int
    title: str
    matrices: Tuple[MatrixSpec, ...]
    m_dtype: str            # storage type of the momentum matrix: 'f32' or 'bf16'
    K: int                  # refresh period (0: never)
    power_iters: int
    steps: int
    grad_kind: str          # 'iid', 'row_scaled', 'layer_std', 'row_col_scaled'
    grad_std: float = 1e-2
    w0_std: float = 1e-2
    beta1: float = 0.9
    beta2: float = 0.999
    eps: float = 1e-8
    lr: float = 1e-3
    capacity_bytes: int = 1 << 29
    grad_layers: int = 28   # layer count spanned by the 'layer_std' gradient scale

    @property
    def params(self) -> int:
        return sum(s.m * s.n for s in self.matrices)

    def subset(self, idx: List[int]) -> "Workload":
        """The same workload restricted to some matrices (parity sampling).

        Each kept matrix keeps its uid, so its draws equal those of the full set.
        """
        return replace(self, matrices=tuple(self.matrices[i] for i in idx))

    def __post_init__(self):
        fixed = tuple(s if s.uid >= 0 else replace(s, uid=i) for i, s in enumerate(self.matrices))
        object.__setattr__(self, "matrices", fixed)


def seed_for(wl_index: int, mat: int, step: int, tag: int) -> int:
    ss = np.random.SeedSequence([int(wl_index), int(mat), int(step), int(tag)])
    return int(ss.generate_state(1, dtype=np.uint64)[0] & ((1 << 63) - 1))


def _log_uniform(rng: np.random.Generator, size: int, lo: float = 1.0, hi: float = 10.0):
    return np.exp(rng.uniform(math.log(lo), math.log(hi), size=size))


# --------------------------------------------------------------------------
# The five workloads
# --------------------------------------------------------------------------

def tiny() -> Workload:
    mats = tuple(MatrixSpec(f"w{i}", 64, 128) for i in range(4))
    return Workload("tiny", 0, "4 fp32 matrices 64x128, refresh every step, 2 power iterations, 3 steps",
                    mats, "f32", K=1, power_iters=2, steps=3, grad_kind="iid", grad_std=1e-2)


def layer(m_dtype: str = "bf16") -> Workload:
    h, f = 1024, 3072
    mats = (MatrixSpec("q", h, h), MatrixSpec("k", h, h), MatrixSpec("v", h, h),
            MatrixSpec("o", h, h), MatrixSpec("up", h, f), MatrixSpec("gate", h, f),
            MatrixSpec("down", f, h))
    return Workload("layer" if m_dtype == "bf16" else "layer_f32m", 1,
                    "one transformer layer, hidden 1024, FFN 3072, refresh every 10 steps, 20 steps",
                    mats, m_dtype, K=10, power_iters=1, steps=20, grad_kind="row_scaled",
                    grad_std=1e-3)


def _qwen_like(hidden: int, kv: int, ffn: int, layers: int):
    mats = []
    for l in range(layers):
        mats += [MatrixSpec(f"l{l}.q", hidden, hidden, l), MatrixSpec(f"l{l}.k", hidden, kv, l),
                 MatrixSpec(f"l{l}.v", hidden, kv, l), MatrixSpec(f"l{l}.o", hidden, hidden, l),
                 MatrixSpec(f"l{l}.up", hidden, ffn, l), MatrixSpec(f"l{l}.gate", hidden, ffn, l),
                 MatrixSpec(f"l{l}.down", ffn, hidden, l)]
    return tuple(mats)


def qwen3_1p7b() -> Workload:
    return Workload("qwen3_1p7b", 2,
                    "Qwen3-1.7B-shaped set: 28 layers x {q,o 2048x2048; k,v 2048x1024; "
                    "up,gate 2048x6144; down 6144x2048}, refresh every 10 steps, 10 steps",
                    _qwen_like(2048, 1024, 6144, 28), "bf16", K=10, power_iters=1, steps=10,
                    grad_kind="layer_std")


_MG_SHAPES = ((4096, 4096), (4096, 1024), (4096, 12288), (12288, 4096))


def microgroup_shapes(seed: int = 0, cap: int = 1 << 29) -> Tuple[Tuple[int, int], ...]:
    """Draw shapes uniformly from the four until nothing more fits the cap.

    A drawn shape is kept when its fp32 gradient payload 4mn still fits the
    remaining capacity; drawing stops once the remainder is smaller than the
    smallest shape.
    """
    rng = np.random.default_rng(seed_for(3, 0, 0, _TAG_SHAPES + seed))
    left = cap
    out = []
    smallest = min(4 * m * n for m, n in _MG_SHAPES)
    guard = 0
    while left >= smallest and guard < 10000:
        guard += 1
        m, n = _MG_SHAPES[int(rng.integers(len(_MG_SHAPES)))]
        if 4 * m * n <= left:
            out.append((m, n))
            left -= 4 * m * n
    return tuple(out)


def microgroup_512mib(seed: int = 0) -> Workload:
    mats = tuple(MatrixSpec(f"g{i}", m, n) for i, (m, n) in enumerate(microgroup_shapes(seed)))
    return Workload("microgroup_512mib", 3,
                    "one 512 MiB-capped micro-group of mixed 4096/1024/12288 shapes, fp32 state, "
                    "refresh every 5 steps with 2 power iterations, 10 steps",
                    mats, "f32", K=5, power_iters=2, steps=10, grad_kind="iid", grad_std=1e-3)


def qwen3_8b_half() -> Workload:
    return Workload("qwen3_8b_half", 4,
                    "Qwen3-8B-shaped matrices at real size, layers 0-17 of 36: "
                    "{q,o 4096x4096; k,v 4096x1024; up,gate 4096x12288; down 12288x4096}, "
                    "refresh every 5 steps, 5 steps",
                    _qwen_like(4096, 1024, 12288, 18), "bf16", K=5, power_iters=1, steps=5,
                    grad_kind="row_col_scaled", grad_std=1e-3)


# Whole-model matrix lists for the cross-rank planners: every matrix of every
# layer, in model order, with one data-parallel bucket per layer (a layer of
# these models holds 48 M (1.7B) or 193 M (8B) parameters, above a typical
# 40 M-parameter gradient bucket, so a bucket never spans two layers).
PLANNING_MODELS = {
    "qwen3_1p7b": (2048, 1024, 6144, 28),
    "qwen3_8b": (4096, 1024, 12288, 36),
}


def planning_set(model: str):
    """(matrices, bucket_begin) of a whole model; bucket b holds matrices
    bucket_begin[b] .. bucket_begin[b+1]-1."""
    hidden, kv, ffn, layers = PLANNING_MODELS[model]
    mats = _qwen_like(hidden, kv, ffn, layers)
    per_layer = len(mats) // layers
    return mats, [per_layer * l for l in range(layers + 1)]


WORKLOADS = {
    "tiny": tiny,
    "layer": layer,
    "layer_f32m": lambda: layer("f32"),
    "qwen3_1p7b": qwen3_1p7b,
    "microgroup_512mib": microgroup_512mib,
    "qwen3_8b_half": qwen3_8b_half,
}


def get(key: str) -> Workload:
    return WORKLOADS[key]()


# --------------------------------------------------------------------------
# Draws (torch, on any device)
# --------------------------------------------------------------------------

def _torch():
    import torch  # deferred so that pure-numpy users need not import torch
    return torch


def _gen(device, seed: int):
    torch = _torch()
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def layer_std(layer_idx: int, layers: int = 28) -> float:
    """Per-layer gradient std spanning 1e-4 .. 1e-2 log-uniformly over the layers."""
    if layers <= 1:
        return 1e-3
    return 10.0 ** (-4.0 + 2.0 * layer_idx / (layers - 1))


def initial_weight(wl: Workload, i: int, device="cpu"):
    torch = _torch()
    s = wl.matrices[i]
    g = _gen(device, seed_for(wl.index, s.uid, 0, _TAG_W0))
    return torch.randn(s.m, s.n, generator=g, device=device, dtype=torch.float32) * wl.w0_std


def _scales(wl: Workload, i: int):
    """Row and column scale vectors drawn once per matrix (numpy, float64)."""
    s = wl.matrices[i]
    rng = np.random.default_rng(seed_for(wl.index, s.uid, 0, _TAG_SCALE))
    r = _log_uniform(rng, s.m)
    c = _log_uniform(rng, s.n)
    return r, c


def gradient(wl: Workload, i: int, t: int, device="cpu"):
    """Gradient of matrix i at step t (t counts from 1), binary32."""
    torch = _torch()
    s = wl.matrices[i]
    g = _gen(device, seed_for(wl.index, s.uid, t, _TAG_G))
    z = torch.randn(s.m, s.n, generator=g, device=device, dtype=torch.float32)
    if wl.grad_kind == "iid":
        return z * wl.grad_std
    if wl.grad_kind == "layer_std":
        return z * layer_std(s.layer, wl.grad_layers)
    r, c = _scales(wl, i)
    if wl.grad_kind == "row_scaled":
        rs = torch.tensor(r * wl.grad_std, dtype=torch.float32, device=device)
        return z * rs[:, None]
    if wl.grad_kind == "row_col_scaled":
        rs = torch.tensor(r * wl.grad_std, dtype=torch.float32, device=device)
        cs = torch.tensor(c, dtype=torch.float32, device=device)
        return z * rs[:, None] * cs[None, :]
    raise ValueError(wl.grad_kind)
