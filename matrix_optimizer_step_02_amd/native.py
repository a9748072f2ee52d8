"""ctypes binding of libmatopt.so (include/matopt.h), argument marshalling only.

Every function here has the name of the C entry point it calls and forwards
plain pointers and sizes; all computation runs in the HIP library. If the
library is missing or fails to load, every call raises: there is no fallback.
"""

from __future__ import annotations

import ctypes as C
import os
from typing import Optional, Sequence

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "_lib", "libmatopt.so")

OPT_OK, OPT_EINVAL, OPT_ENOWS, OPT_EHIP, OPT_EUNSUPPORTED, OPT_ESTATE = 0, -1, -2, -3, -4, -5
OPT_F32, OPT_BF16 = 0, 1
OPT_FLAG_ROTATED_MOMENTUM = 1
OPT_FLAG_BF16_ROTATION = 2
OPT_FLAG_MUON = 4
OPT_FLAG_FP32_MFMA = 8
OPT_FLAG_BF16_BASES = 16
OPT_MAX_DIM = 16384
OPT_STATIC_MAX_DIM = 4096
PHASES = ("momentum", "refresh", "rot_left", "rot_right", "adam", "back_left", "back_right", "ortho", "rot_pieced")
OPT_NUM_PHASES = len(PHASES)

EXPORTED = (
    "opt_group_workspace_size", "opt_group_create", "opt_group_step", "opt_group_refresh_basis",
    "opt_group_get_step", "opt_group_set_step", "opt_group_set_lr", "opt_plan",
    "opt_group_set_timing", "opt_group_read_timing", "opt_group_destroy", "opt_last_error",
    "opt_gemm", "opt_gemm_x6", "opt_gemm_bf16", "opt_orthonormalize_workspace_size", "opt_orthonormalize",
    "opt_partition_dp", "opt_plan_host_ranks", "opt_group_health", "opt_group_reorthonormalize",
    "opt_orthonormalize_static", "opt_group_read_group_timing", "opt_group_workspace_parts",
)


class MatoptError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"matopt status {status}: {msg}")
        self.status = status


class opt_matrix_desc(C.Structure):
    _fields_ = [
        ("m", C.c_int64), ("n", C.c_int64),
        ("W", C.c_void_p), ("G", C.c_void_p), ("M", C.c_void_p), ("M_dtype", C.c_int32),
        ("v", C.c_void_p), ("U", C.c_void_p), ("V", C.c_void_p), ("Mt", C.c_void_p),
    ]


class opt_hparams(C.Structure):
    _fields_ = [
        ("beta1", C.c_float), ("beta2", C.c_float), ("eps", C.c_float), ("lr", C.c_float),
        ("K", C.c_int32), ("power_iters", C.c_int32),
        ("capacity_bytes", C.c_uint64), ("refresh_capacity_bytes", C.c_uint64), ("flags", C.c_uint32),
        ("ns_iters", C.c_int32),
    ]


class opt_health(C.Structure):
    _fields_ = [
        ("orth_U", C.c_double), ("orth_V", C.c_double), ("v_mean_abs", C.c_double), ("v_std", C.c_double),
        ("v_min", C.c_double), ("v_max", C.c_double), ("nonfinite", C.c_int64),
    ]


_lib: Optional[C.CDLL] = None


def load(path: str = LIB_PATH) -> C.CDLL:
    """Load the library once. torch is imported first so that the HIP runtime
    it ships is the one the library binds to (same soname)."""
    global _lib
    if _lib is not None:
        return _lib
    import torch  # noqa: F401  (binds libamdhip64 before the library is loaded)
    if not os.path.exists(path):
        raise MatoptError(OPT_ESTATE, f"{path} is missing: run __graft_entry__.build() first")
    lib = C.CDLL(path)
    vp, i32, i64, u64, f32 = C.c_void_p, C.c_int32, C.c_int64, C.c_uint64, C.c_float
    D, H = C.POINTER(opt_matrix_desc), C.POINTER(opt_hparams)
    sig = {
        "opt_group_workspace_size": ([D, i32, H, C.POINTER(u64)], i32),
        "opt_group_workspace_parts": ([D, i32, H, C.POINTER(u64)], i32),
        "opt_group_create": ([D, i32, H, vp, u64, vp, C.POINTER(vp)], i32),
        "opt_group_step": ([vp, vp], i32),
        "opt_group_refresh_basis": ([vp, i32, vp], i32),
        "opt_group_get_step": ([vp, C.POINTER(i64)], i32),
        "opt_group_set_step": ([vp, i64], i32),
        "opt_group_set_lr": ([vp, f32], i32),
        "opt_plan": ([D, i32, H, C.POINTER(i32), C.POINTER(i32), C.POINTER(i32)], i32),
        "opt_group_set_timing": ([vp, i32], i32),
        "opt_group_read_timing": ([vp, C.POINTER(C.c_double), C.POINTER(i64)], i32),
        "opt_group_destroy": ([vp], None),
        "opt_last_error": ([], C.c_char_p),
        "opt_gemm": ([i32, i32, i64, i64, i64, f32, vp, i32, i64, vp, i32, i64, f32, vp, i64, vp], i32),
        "opt_gemm_x6": ([i32, i32, i64, i64, i64, f32, vp, i32, i64, vp, i32, i64, f32, vp, i64, vp], i32),
        "opt_gemm_bf16": ([i64, i64, i64, f32, vp, i64, vp, i64, f32, vp, i32, i64, vp], i32),
        "opt_orthonormalize_workspace_size": ([i64, C.POINTER(u64)], i32),
        "opt_orthonormalize": ([vp, vp, i64, vp, u64, vp], i32),
        "opt_orthonormalize_static": ([vp, vp, i64, vp], i32),
        "opt_group_read_group_timing": ([vp, C.POINTER(C.c_double), i32], i32),
        "opt_group_health": ([vp, C.POINTER(opt_health), vp], i32),
        "opt_group_reorthonormalize": ([vp, i32, vp], i32),
        "opt_partition_dp": ([C.POINTER(C.c_double), i64, C.POINTER(i64), i32, i32, C.c_double,
                              C.POINTER(i32), C.POINTER(C.c_double)], i32),
        "opt_plan_host_ranks": ([C.POINTER(C.c_double), C.POINTER(u64), i64, i32, u64, C.POINTER(i32),
                                 C.POINTER(i32), C.POINTER(i32), C.POINTER(i32)], i32),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib


def _check(st: int):
    if st != OPT_OK:
        raise MatoptError(st, load().opt_last_error().decode(errors="replace"))


def _descs(descs: Sequence[opt_matrix_desc]):
    arr = (opt_matrix_desc * len(descs))(*descs)
    return arr, len(descs)


def opt_last_error() -> str:
    return load().opt_last_error().decode(errors="replace")


def opt_group_workspace_size(descs, hp: opt_hparams) -> int:
    arr, n = _descs(descs)
    out = C.c_uint64(0)
    _check(load().opt_group_workspace_size(arr, n, C.byref(hp), C.byref(out)))
    return out.value


def opt_group_workspace_parts(descs, hp: opt_hparams) -> dict:
    """The workspace's parts in bytes: work lists, copies of the bases, step
    scratch and the largest refresh batch (which overlays the two before)."""
    arr, n = _descs(descs)
    out = (C.c_uint64 * 4)()
    _check(load().opt_group_workspace_parts(arr, n, C.byref(hp), out))
    return dict(zip(("tables", "copies", "scratch", "refresh"), (int(x) for x in out)))


def opt_group_create(descs, hp: opt_hparams, workspace_ptr: int, workspace_bytes: int,
                     stream_ptr: int) -> int:
    arr, n = _descs(descs)
    out = C.c_void_p(0)
    _check(load().opt_group_create(arr, n, C.byref(hp), C.c_void_p(workspace_ptr), workspace_bytes,
                                   C.c_void_p(stream_ptr), C.byref(out)))
    return out.value


def opt_group_step(g: int, stream_ptr: int):
    _check(load().opt_group_step(C.c_void_p(g), C.c_void_p(stream_ptr)))


def opt_group_refresh_basis(g: int, power_iters: int, stream_ptr: int):
    _check(load().opt_group_refresh_basis(C.c_void_p(g), power_iters, C.c_void_p(stream_ptr)))


def opt_group_get_step(g: int) -> int:
    t = C.c_int64(0)
    _check(load().opt_group_get_step(C.c_void_p(g), C.byref(t)))
    return t.value


def opt_group_set_step(g: int, t: int):
    _check(load().opt_group_set_step(C.c_void_p(g), t))


def opt_group_set_lr(g: int, lr: float):
    _check(load().opt_group_set_lr(C.c_void_p(g), lr))


def opt_plan(descs, hp: opt_hparams):
    """Returns (order, group_of, num_groups) of the micro-group planner."""
    arr, n = _descs(descs)
    order = (C.c_int32 * n)()
    group_of = (C.c_int32 * n)()
    ng = C.c_int32(0)
    _check(load().opt_plan(arr, n, C.byref(hp), order, group_of, C.byref(ng)))
    return list(order), list(group_of), ng.value


def opt_group_health(g: int, count: int, stream_ptr: int):
    """Returns a list of dicts (one per matrix, input order)."""
    out = (opt_health * count)()
    _check(load().opt_group_health(C.c_void_p(g), out, C.c_void_p(stream_ptr)))
    return [{f: getattr(h, f) for f, _ in opt_health._fields_} for h in out]


def opt_group_reorthonormalize(g: int, iters: int, stream_ptr: int):
    _check(load().opt_group_reorthonormalize(C.c_void_p(g), iters, C.c_void_p(stream_ptr)))


def opt_group_set_timing(g: int, enable: bool):
    _check(load().opt_group_set_timing(C.c_void_p(g), 1 if enable else 0))


def opt_group_read_group_timing(g: int, ngroups: int):
    """Summed milliseconds of each micro-group's timed scopes."""
    ms = (C.c_double * max(ngroups, 1))()
    _check(load().opt_group_read_group_timing(C.c_void_p(g), ms, ngroups))
    return list(ms)[:ngroups]


def opt_group_read_timing(g: int):
    ms = (C.c_double * OPT_NUM_PHASES)()
    cnt = (C.c_int64 * OPT_NUM_PHASES)()
    _check(load().opt_group_read_timing(C.c_void_p(g), ms, cnt))
    return {PHASES[i]: (ms[i], cnt[i]) for i in range(OPT_NUM_PHASES)}


def opt_group_destroy(g: int):
    if g:
        load().opt_group_destroy(C.c_void_p(g))


def opt_gemm(trans_a: int, trans_b: int, M: int, N: int, K: int, alpha: float, A: int, a_dtype: int,
             lda: int, B: int, b_dtype: int, ldb: int, beta: float, Cp: int, ldc: int, stream_ptr: int):
    _check(load().opt_gemm(trans_a, trans_b, M, N, K, alpha, C.c_void_p(A), a_dtype, lda,
                           C.c_void_p(B), b_dtype, ldb, beta, C.c_void_p(Cp), ldc,
                           C.c_void_p(stream_ptr)))


def opt_gemm_x6(trans_a: int, trans_b: int, M: int, N: int, K: int, alpha: float, A: int, a_dtype: int,
                lda: int, B: int, b_dtype: int, ldb: int, beta: float, Cp: int, ldc: int, stream_ptr: int):
    _check(load().opt_gemm_x6(trans_a, trans_b, M, N, K, alpha, C.c_void_p(A), a_dtype, lda,
                              C.c_void_p(B), b_dtype, ldb, beta, C.c_void_p(Cp), ldc,
                              C.c_void_p(stream_ptr)))


def opt_gemm_bf16(M: int, N: int, K: int, alpha: float, A: int, lda: int, B: int, ldb: int, beta: float,
                  Cp: int, c_dtype: int, ldc: int, stream_ptr: int):
    _check(load().opt_gemm_bf16(M, N, K, alpha, C.c_void_p(A), lda, C.c_void_p(B), ldb, beta, C.c_void_p(Cp),
                                c_dtype, ldc, C.c_void_p(stream_ptr)))


def opt_orthonormalize_workspace_size(d: int) -> int:
    out = C.c_uint64(0)
    _check(load().opt_orthonormalize_workspace_size(d, C.byref(out)))
    return out.value


def opt_orthonormalize(Z: int, Q: int, d: int, workspace: int, workspace_bytes: int, stream_ptr: int):
    _check(load().opt_orthonormalize(C.c_void_p(Z), C.c_void_p(Q), d, C.c_void_p(workspace),
                                     workspace_bytes, C.c_void_p(stream_ptr)))


def opt_orthonormalize_static(Z: int, Q: int, d: int, stream_ptr: int):
    _check(load().opt_orthonormalize_static(C.c_void_p(Z), C.c_void_p(Q), d, C.c_void_p(stream_ptr)))


def opt_partition_dp(cost: Sequence[float], bucket_begin: Sequence[int], ranks: int, alpha: float):
    """Returns (owner per parameter, load per rank)."""
    n, nb = len(cost), len(bucket_begin) - 1
    c = (C.c_double * max(n, 1))(*cost)
    bb = (C.c_int64 * len(bucket_begin))(*bucket_begin)
    owner = (C.c_int32 * max(n, 1))()
    loads = (C.c_double * ranks)()
    _check(load().opt_partition_dp(c, n, bb, nb, ranks, alpha, owner, loads))
    return list(owner)[:n], list(loads)


def opt_plan_host_ranks(cost: Sequence[float], nbytes: Sequence[int], ranks: int, capacity_bytes: int):
    """Returns (order, group_of, host_of, num_groups)."""
    n = len(cost)
    c = (C.c_double * max(n, 1))(*cost)
    b = (C.c_uint64 * max(n, 1))(*nbytes)
    order = (C.c_int32 * max(n, 1))()
    group_of = (C.c_int32 * max(n, 1))()
    host_of = (C.c_int32 * max(n, 1))()
    ng = C.c_int32(0)
    _check(load().opt_plan_host_ranks(c, b, n, ranks, capacity_bytes, order, group_of, host_of,
                                          C.byref(ng)))
    return list(order)[:n], list(group_of)[:n], list(host_of)[:n], ng.value
