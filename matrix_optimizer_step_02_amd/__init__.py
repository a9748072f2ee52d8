"""MI355X (gfx950) rotated-basis matrix-optimizer step.

The compute path is libmatopt.so (HIP kernels behind a C ABI, include/matopt.h).
This package only marshals torch tensors (device memory and streams) into the
C ABI: ``native`` mirrors the C entry points one to one, ``RotatedAdamGroup``
holds the descriptors and the workspace of one group of matrices.
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import List, Optional, Sequence

from . import native
from .native import MatoptError, OPT_BF16, OPT_F32, PHASES  # noqa: F401

__all__ = ["RotatedAdamGroup", "Hyper", "MatoptError", "native", "tensor_ptr", "stream_ptr"]


@dataclass
class Hyper:
    beta1: float = 0.9
    beta2: float = 0.999
    eps: float = 1e-8
    lr: float = 1e-3
    K: int = 10
    power_iters: int = 1
    capacity_bytes: int = 1 << 29
    refresh_capacity_bytes: int = 0   # 0: library default (48 GiB)
    rotated_momentum: bool = False    # carry m~ in rotated coordinates (needs an Mt tensor per matrix)
    bf16_rotation: bool = False       # rotations on bf16 operands (fp32 accumulation) from the second step
    muon: bool = False                # orthogonalised-momentum step instead (no v, U, V)
    ns_iters: int = 0                 # Newton-Schulz iterations of the muon step (>= 1 there)
    fp32_mfma: bool = False           # keep the fp32 products on fp32 MFMAs (no bf16-piece products)
    bf16_bases: bool = False          # U, V stored in bf16 only (with bf16_rotation)

    def c(self) -> native.opt_hparams:
        flags = (native.OPT_FLAG_ROTATED_MOMENTUM if self.rotated_momentum else 0) | \
                (native.OPT_FLAG_BF16_ROTATION if self.bf16_rotation else 0) | \
                (native.OPT_FLAG_MUON if self.muon else 0) | \
                (native.OPT_FLAG_FP32_MFMA if self.fp32_mfma else 0) | \
                (native.OPT_FLAG_BF16_BASES if self.bf16_bases else 0)
        return native.opt_hparams(self.beta1, self.beta2, self.eps, self.lr, self.K,
                                  self.power_iters, self.capacity_bytes,
                                  self.refresh_capacity_bytes, flags, self.ns_iters)


def tensor_ptr(t) -> int:
    return int(t.data_ptr())


def stream_ptr(stream=None) -> int:
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return int(s.cuda_stream)


def _check_tensor(t, shape, dtypes, name, device):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype not in dtypes:
        raise ValueError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous (row-major)")


def make_desc(W, G, M, v, U, V, Mt=None) -> native.opt_matrix_desc:
    """Descriptor of one matrix from torch tensors on one HIP device (Mt: the
    rotated momentum, only with Hyper.rotated_momentum)."""
    import torch
    m, n = W.shape
    dev = W.device
    if dev.type != "cuda":
        raise ValueError("tensors must live on a HIP device")
    _check_tensor(W, (m, n), (torch.float32,), "W", dev)
    _check_tensor(G, (m, n), (torch.float32,), "G", dev)
    _check_tensor(M, (m, n), (torch.float32, torch.bfloat16), "M", dev)
    if v is not None:
        _check_tensor(v, (m, n), (torch.float32,), "v", dev)
    for t, shape, name in ((U, (m, m), "U"), (V, (n, n), "V")):
        if t is not None:   # absent only for the muon step; bf16 for bases stored in 16 bits
            _check_tensor(t, shape, (torch.float32, torch.bfloat16), name, dev)
    if Mt is not None:
        _check_tensor(Mt, (m, n), (torch.float32,), "Mt", dev)
    dt = native.OPT_BF16 if M.dtype == torch.bfloat16 else native.OPT_F32
    return native.opt_matrix_desc(m, n, tensor_ptr(W), tensor_ptr(G), tensor_ptr(M), dt,
                                  *(tensor_ptr(t) if t is not None else 0 for t in (v, U, V)),
                                  tensor_ptr(Mt) if Mt is not None else 0)


class RotatedAdamGroup:
    """A group of whole matrices stepped together by the HIP library.

    ``params`` is a sequence of dicts with tensors W, G, M, v, U, V (all
    caller-owned, kept referenced here). The caller writes each step's
    gradient into G before calling :meth:`step`.
    """

    def __init__(self, params: Sequence[dict], hp: Hyper, stream=None):
        import torch
        self.params = list(params)
        self.hp = hp
        want = torch.bfloat16 if hp.bf16_bases else torch.float32
        for p in self.params:
            for key in ("U", "V"):
                if p.get(key) is not None and p[key].dtype != want:
                    raise ValueError(f"{key} must be {want} (bf16_bases={hp.bf16_bases})")
        self.descs = [make_desc(p["W"], p["G"], p["M"], p.get("v"), p.get("U"), p.get("V"), p.get("Mt"))
                      for p in self.params]
        self._hpc = hp.c()
        self.ws_bytes = native.opt_group_workspace_size(self.descs, self._hpc)
        dev = self.params[0]["W"].device
        self.workspace = torch.empty(max(self.ws_bytes, 256), dtype=torch.uint8, device=dev)
        self._g = native.opt_group_create(self.descs, self._hpc, tensor_ptr(self.workspace),
                                          self.workspace.numel(), stream_ptr(stream))

    @staticmethod
    def plan(shapes: Sequence[tuple], hp: Hyper):
        descs = [native.opt_matrix_desc(m, n, 0, 0, 0, 0, 0, 0, 0, 0) for (m, n) in shapes]
        return native.opt_plan(descs, hp.c())

    def step(self, stream=None):
        native.opt_group_step(self._g, stream_ptr(stream))

    def refresh_basis(self, power_iters: Optional[int] = None, stream=None):
        native.opt_group_refresh_basis(self._g, power_iters or self.hp.power_iters, stream_ptr(stream))

    @property
    def t(self) -> int:
        return native.opt_group_get_step(self._g)

    @t.setter
    def t(self, value: int):
        native.opt_group_set_step(self._g, value)

    def set_lr(self, lr: float):
        native.opt_group_set_lr(self._g, lr)
        self.hp.lr = lr

    def health(self, stream=None):
        """Per-matrix state checks: orthogonality drift of U and V, statistics
        of v, non-finite count of W, M, v (synchronises the stream)."""
        return native.opt_group_health(self._g, len(self.descs), stream_ptr(stream))

    def reorthonormalize(self, iters: int = 1, stream=None):
        native.opt_group_reorthonormalize(self._g, iters, stream_ptr(stream))

    def set_timing(self, enable: bool):
        native.opt_group_set_timing(self._g, enable)

    def read_timing(self):
        return native.opt_group_read_timing(self._g)

    def read_group_timing(self):
        """Summed milliseconds of each micro-group's timed scopes (plan order)."""
        _, _, ngroups = RotatedAdamGroup.plan([(int(d.m), int(d.n)) for d in self.descs], self.hp)
        return native.opt_group_read_group_timing(self._g, ngroups)

    def close(self):
        if getattr(self, "_g", None):
            native.opt_group_destroy(self._g)
            self._g = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def new_state(m: int, n: int, m_dtype: str = "f32", device="cuda", W0=None, rotated_momentum=False,
              bases=True, bases16=False):
    """Fresh caller-side state of one matrix: W (given or zeros), G zeros,
    M and v zeros, U = I_m, V = I_n (bf16 with bases16) (and Mt,
    uninitialised, for the rotated momentum). bases=False leaves out v, U
    and V (the muon step)."""
    import torch
    dt = torch.bfloat16 if m_dtype == "bf16" else torch.float32
    W = (W0.to(device=device, dtype=torch.float32).contiguous().clone() if W0 is not None
         else torch.zeros(m, n, device=device))
    st = {
        "W": W,
        "G": torch.zeros(m, n, device=device),
        "M": torch.zeros(m, n, device=device, dtype=dt),
    }
    if bases:
        bdt = torch.bfloat16 if bases16 else torch.float32
        st |= {"v": torch.zeros(m, n, device=device), "U": torch.eye(m, device=device, dtype=bdt),
               "V": torch.eye(n, device=device, dtype=bdt)}
    return st | ({"Mt": torch.empty(m, n, device=device)} if rotated_momentum else {})
