"""Benchmark of the rotated-basis matrix-optimizer step on one MI355X.

    python bench.py [--gpus 1] [--steps 10] [--warmup 2] [--workload qwen3_1p7b]

One step is one pass of the whole hot path over every matrix of the workload:
momentum EMA, the basis refresh when due (t = 1, K+1, ...), the two-sided
rotations, the rotated Adam moments, the rotation back and the weight update.
The gradient of step 1 is drawn once before the timed region and stays
resident in the gradient buffers (the optimizer reads them each step; the
values do not change the work done). With the default 2 warm-up steps the 10
timed steps are t = 3..12 and include exactly one refresh (t = 11), the
workload's own cadence of one refresh per 10 steps.

Prints one JSON line. `value` is parameters updated per second (sum of m*n
over the matrices times steps per second). `roofline` is for the rotation
GEMMs (the dominant kernels), timed with HIP events recorded by the library
on the step's stream around every launch of each phase inside the timed
region. `cpu_baseline` times the fp64 oracle on a bounded sample (see
--cpu-sample-s), on rank 0 only.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

MI355X_FP32_MFMA_TFLOPS = 157.3
MI355X_BF16_MFMA_TFLOPS = 2500.0   # dense bf16 MFMA (no sparsity)
MI355X_HBM_GBPS = 8000.0
# ceiling of an fp32 product done as six bf16 MFMA products (three-piece split)
X6_FP32_EQUIV_TFLOPS = MI355X_BF16_MFMA_TFLOPS / 6
TRAFFIC_JSON = os.path.join(ROOT, "profiles", "rotation_gemm_traffic.json")
# the kernel's sources and the schedule that decides what each launch holds
GEMM_SOURCES = ("matrix_optimizer_step_02_amd/csrc/gemm.hip", "matrix_optimizer_step_02_amd/csrc/gemm.h",
                "matrix_optimizer_step_02_amd/csrc/gmem.h", "matrix_optimizer_step_02_amd/csrc/api.hip")
def is_rotation_gemm(kernel_name: str) -> bool:
    """Any instantiation of the grouped GEMM (fp32 MFMAs, or the fp32
    products on bf16 MFMAs): in a step without a refresh every one of its
    launches is a rotation phase."""
    return "gemm_grouped_kernel<" in kernel_name or "gemm_x6_kernel<" in kernel_name

METRIC = "optimizer steps/s + params updated/s per micro-group; HBM GB/s & MFMA util"


def rotation_flops(shapes):
    return sum(6.0 * m * n * (m + n) for m, n in shapes)


def pieced(m, n, m_dtype, no_flags):
    """Whether the library runs this matrix's momentum product U^T M (m > n)
    or M V (else) as three bf16 products against exact pieces of the basis:
    fp32 rotations of a bf16 M with m, n multiples of 8."""
    return no_flags and m_dtype == "bf16" and m % 8 == 0 and n % 8 == 0


def phase_flops(shapes, carry=False, m_dtype="f32", no_flags=False):
    """Algorithmic flops of each GEMM phase for one step over all matrices
    (carry: a step of the rotated-momentum variant that rotates G alone;
    no_flags: the method's fp32 rotations with no flag, where a bf16 M's
    larger product moves to the pieced phase)."""
    out = {"rot_left": 0.0, "rot_right": 0.0, "back_left": 0.0, "back_right": 0.0}
    for m, n in shapes:
        out["rot_left"] += 2.0 * m * m * n
        out["rot_right"] += 2.0 * m * n * n
        out["back_left"] += 2.0 * m * m * n
        out["back_right"] += 2.0 * m * n * n
        if carry:
            continue
        if pieced(m, n, m_dtype, no_flags):
            # U^T M (tall) or M V (wide/square) pieced, the other product fp32
            out["rot_pieced"] = out.get("rot_pieced", 0.0) + 2.0 * m * n * max(m, n)
            out["rot_right" if m > n else "rot_left"] += 2.0 * m * n * min(m, n)
        else:
            out["rot_left"] += 2.0 * m * m * n
            out["rot_right"] += 2.0 * m * n * n
    return out


def elementwise_bytes(shapes, m_dtype):
    mb = 2 if m_dtype == "bf16" else 4
    mn = sum(m * n for m, n in shapes)
    return {"momentum": mn * (4 + 2 * mb), "adam": mn * 20.0}


def gemm_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for rel in GEMM_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def rotation_dispatches(rows):
    """The rotation-GEMM dispatches among profiled kernels: a step starts with
    its run of momentum kernels; the refresh's Gram products and QR block
    updates use the same GEMM instantiations as the rotations, so only steps
    without a refresh (no QR kernel) are taken, and there every grouped GEMM
    is a rotation phase."""
    rows = sorted(rows, key=lambda r: int(r["Dispatch_Id"]))
    steps, cur = [], None
    for r in rows:
        name = r["Kernel_Name"]
        if "momentum_kernel" in name:
            if cur is None or cur["other"]:
                cur = {"rows": [], "refresh": False, "other": False}
                steps.append(cur)
        elif cur is not None:
            cur["other"] = True
        if cur is None:
            continue
        cur["rows"].append(r)
        if "qr_" in name or "copy_cols" in name:
            cur["refresh"] = True
    return [r for st in steps if not st["refresh"] for r in st["rows"] if is_rotation_gemm(r["Kernel_Name"])]


def summarize_pmc(fetch_csv: str, write_csv: str, calib_mib: int, out_path: str = TRAFFIC_JSON):
    """HBM bytes per rotation-GEMM launch from two rocprofv3 --pmc runs.

    Each counter is scaled by what it reads for the calibration copy (the
    first __amd_rocclr_copyBuffer dispatch, `calib_mib` MiB read and written).
    """
    import csv
    def rows(path, counter):
        with open(path) as f:
            return [r for r in csv.DictReader(f) if r["Counter_Name"] == counter]
    F, W = rows(fetch_csv, "FETCH_SIZE"), rows(write_csv, "WRITE_SIZE")
    calib = calib_mib * (1 << 20)
    cf = float(next(r for r in F if "copyBuffer" in r["Kernel_Name"])["Counter_Value"]) * 1024
    cw = float(next(r for r in W if "copyBuffer" in r["Kernel_Name"])["Counter_Value"]) * 1024
    sf, sw = calib / cf, calib / cw
    fr = [float(r["Counter_Value"]) * 1024 * sf for r in rotation_dispatches(F)]
    wr = [float(r["Counter_Value"]) * 1024 * sw for r in rotation_dispatches(W)]
    out = {
        "kernel": "gemm_x6_kernel (and gemm_grouped_kernel), rotation-phase instantiations",
        "gemm_source_sha256": gemm_source_hash(),
        "launches": len(fr),
        "fetch_bytes_per_launch": sum(fr) / len(fr),
        "write_bytes_per_launch": sum(wr) / len(wr),
        "fetch_scale": sf, "write_scale": sw,
        "calibration": f"{calib_mib} MiB device copy (__amd_rocclr_copyBuffer): FETCH_SIZE x{sf:.4f}, "
                       f"WRITE_SIZE x{sw:.4f}",
    }
    with open(out_path, "w") as f:
        json.dump(out, f, indent=1)
    return out


def traffic_per_launch():
    """Counter bytes per rotation-GEMM launch, or None if the GEMM source has
    changed since the counters were taken."""
    try:
        with open(TRAFFIC_JSON) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("gemm_source_sha256") != gemm_source_hash():
        return None
    return t["fetch_bytes_per_launch"] + t["write_bytes_per_launch"]


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def refresh_flops(m: int, n: int, p: int) -> float:
    """Algorithmic flops of one refresh of an m x n matrix with p passes."""
    return p * (8.0 * m * n * min(m, n) + (8.0 / 3.0) * (float(m) ** 3 + float(n) ** 3))


def cpu_baseline(wl, budget_s: float, muon_iters: int = 0):
    """The oracle as it stands, timed on the host: one non-refresh step on
    one matrix of each distinct shape, and (for the method) one refresh step
    on the shapes whose refresh fits the remaining budget, the others
    estimated from the measured refresh rate (flops/s of the oracle's
    refresh on the largest shape timed); combined at the workload's cadence
    of one refresh per K steps, weighted by shape counts, scaled to
    parameters/s (muon_iters > 0: the orthogonalised-momentum oracle)."""
    import numpy as np
    import oracle
    import workloads
    import threadpoolctl  # noqa: F401  (reports BLAS threads)
    from collections import Counter
    counts = Counter((s.m, s.n) for s in wl.matrices)
    hp = oracle.Hyper(wl.beta1, wl.beta2, wl.eps, wl.lr, 0, wl.power_iters)
    total_s = 0.0
    done = []
    t_start = time.time()
    for (m, n), c in sorted(counts.items(), key=lambda kv: kv[0][0] * kv[0][1]):
        if time.time() - t_start > budget_s:
            break
        i = next(k for k, s in enumerate(wl.matrices) if (s.m, s.n) == (m, n))
        st = oracle.OracleState.fresh(workloads.initial_weight(wl, i).double().numpy(), wl.m_dtype)
        G = workloads.gradient(wl, i, 1).double().numpy()
        # basis from an earlier refresh: the identity is as costly for the oracle as any other
        t0 = time.time()
        if muon_iters:
            from oracle import muon
            muon.muon_apply(st.W, st.M, G, wl.beta1, wl.lr, muon_iters, wl.m_dtype)
        else:
            oracle.step(st, G, hp)
        dt = time.time() - t0
        total_s += dt * c
        done.append((m, n, c, dt))
    covered = sum(m * n * c for m, n, c, _ in done)
    threads = None
    try:
        from threadpoolctl import threadpool_info
        threads = max((x.get("num_threads") or 0) for x in threadpool_info()) or None
    except Exception:
        pass
    plain_value = covered / total_s if total_s > 0 else None
    out = {
        "value": plain_value,
        "unit": "params/s",
        "cores": threads or os.cpu_count(),
        "kind": "oracle",
        "cpu_model": cpu_model(),
        "host_cpus": os.cpu_count(),
    }
    if muon_iters or wl.K <= 0:
        out["sample"] = ((f"one fp64 orthogonalised-momentum oracle step ({muon_iters} Newton-Schulz iterations)"
                          if muon_iters else "one fp64 oracle step")
                         + " on one matrix of each distinct shape "
                         + ", ".join(f"{m}x{n} ({dt:.2f} s, x{c})" for m, n, c, dt in done))
        return out
    # refresh steps: time one on the smaller shapes while the budget lasts
    hp_r = oracle.Hyper(wl.beta1, wl.beta2, wl.eps, wl.lr, 1, wl.power_iters)
    refresh_s = {}
    for (m, n), c in sorted(counts.items(), key=lambda kv: refresh_flops(*kv[0], wl.power_iters)):
        est = None
        if refresh_s:
            (m0, n0), t0r = max(refresh_s.items(), key=lambda kv: refresh_flops(*kv[0], wl.power_iters))
            est = t0r * refresh_flops(m, n, wl.power_iters) / refresh_flops(m0, n0, wl.power_iters)
        if time.time() - t_start + (est or 0.0) > 3 * budget_s:
            break
        i = next(k for k, s in enumerate(wl.matrices) if (s.m, s.n) == (m, n))
        st = oracle.OracleState.fresh(workloads.initial_weight(wl, i).double().numpy(), wl.m_dtype)
        G = workloads.gradient(wl, i, 1).double().numpy()
        t0 = time.time()
        oracle.step(st, G, hp_r)          # t = 1: refresh, then the rotations
        refresh_s[(m, n)] = time.time() - t0
    if not refresh_s or len(done) < len(counts):
        out["sample"] = "incomplete: the budget ran out before every shape was timed"
        return out
    (mr, nr), tr = max(refresh_s.items(), key=lambda kv: refresh_flops(*kv[0], wl.power_iters))
    rate = refresh_flops(mr, nr, wl.power_iters) / tr      # oracle refresh flops/s on the largest timed shape
    plain = {(m, n): dt for m, n, c, dt in done}
    total = 0.0
    parts = []
    for (m, n), c in counts.items():
        t_ref = refresh_s.get((m, n))
        measured = t_ref is not None
        if not measured:
            t_ref = plain[(m, n)] + refresh_flops(m, n, wl.power_iters) / rate
        total += c * ((wl.K - 1) * plain[(m, n)] + t_ref) / wl.K
        parts.append(f"{m}x{n} x{c}: plain {plain[(m, n)]:.2f} s, refresh step {t_ref:.2f} s"
                     + ("" if measured else " (estimated)"))
    out["value"] = covered / total
    out["plain_steps_value"] = plain_value
    out["refresh_step_s"] = {f"{m}x{n}": t for (m, n), t in refresh_s.items()}
    out["sample"] = ("fp64 oracle steps on one matrix of each distinct shape, combined at one refresh step per "
                     f"K = {wl.K} steps: " + "; ".join(parts)
                     + f". Refresh steps not timed are estimated from the oracle's refresh rate on {mr}x{nr} "
                       f"({rate / 1e9:.1f} GFLOP/s); its unblocked QR runs slower at larger orders, so the "
                       "estimate over-states the oracle's rate")
    return out


def time_orthonormalize(orders) -> int:
    """One JSON line per order: opt_orthonormalize of a seeded Gaussian
    d x d matrix, three runs (the first includes one-time set-up), with the
    orthonormality of the result."""
    import torch
    import matrix_optimizer_step_02_amd as mo
    N = mo.native
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    for d in orders:
        g = torch.Generator().manual_seed(d)
        Z0 = torch.randn(d, d, generator=g).to("cuda")
        Q = torch.empty_like(Z0)
        nb = N.opt_orthonormalize_workspace_size(d)
        ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
        times = []
        for _ in range(3):
            Z = Z0.clone()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            N.opt_orthonormalize(Z.data_ptr(), Q.data_ptr(), d, ws.data_ptr(), nb, mo.stream_ptr())
            e1.record()
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
        orth = float((Q.T @ Q - torch.eye(d, device="cuda")).abs().max())
        print(json.dumps({"orthonormalize": d, "ms": times, "flops": (8.0 / 3.0) * d ** 3,
                          "tflops": (8.0 / 3.0) * d ** 3 / (min(times) * 1e-3) / 1e12, "orth": orth}), flush=True)
    return 0


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="qwen3_1p7b")
    ap.add_argument("--cpu-sample-s", type=float, default=30.0,
                    help="budget for the oracle CPU baseline (0 disables it)")
    ap.add_argument("--no-timing", action="store_true", help="do not record per-phase HIP events")
    ap.add_argument("--rotated-momentum", action="store_true",
                    help="the variant that carries m~ in rotated coordinates within a basis epoch")
    ap.add_argument("--bf16-rotation", action="store_true",
                    help="the variant that runs the rotations on bf16 operands (fp32 accumulation)")
    ap.add_argument("--bf16-bases", action="store_true",
                    help="with --bf16-rotation: U and V stored in bf16 only (the refresh widens and rounds them)")
    ap.add_argument("--muon", action="store_true",
                    help="the orthogonalised-momentum step (Newton-Schulz polar factor of M) instead")
    ap.add_argument("--ns-iters", type=int, default=5, help="Newton-Schulz iterations of --muon")
    ap.add_argument("--fp32-mfma", action="store_true",
                    help="keep the fp32 products on fp32 MFMAs (no bf16-piece products)")
    ap.add_argument("--compare-single", action="store_true",
                    help="also time one plain product of the same flop count as an average rotation launch "
                         "(opt_gemm_x6, square, fp32 operands) to compare the grouped launches' rate with")
    ap.add_argument("--refresh-cap-gib", type=float, default=0.0,
                    help="scratch cap of one refresh batch in GiB (0: the library default)")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="run a plain device copy of this many MiB first (a dispatch of known size "
                         "for scaling hardware byte counters)")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write the rotation-GEMM traffic summary from two rocprofv3 --pmc "
                         "counter_collection.csv files (FETCH_SIZE, WRITE_SIZE) and exit")
    ap.add_argument("--orthonormalize", type=int, nargs="+", metavar="D",
                    help="instead of the step: time opt_orthonormalize (the refresh's QR) on one "
                         "seeded d x d Gaussian matrix per order D, three runs each, and exit")
    args = ap.parse_args(argv)
    if args.orthonormalize:
        return time_orthonormalize(args.orthonormalize)
    if args.summarize_pmc:
        print(json.dumps(summarize_pmc(*args.summarize_pmc, calib_mib=args.calibrate_copy_mib or 1024)))
        return 0

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path "
              "(the step shards by whole matrix; see the design notes)", file=sys.stderr)
        return 2

    import torch
    import matrix_optimizer_step_02_amd as mo
    import workloads

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wl = workloads.get(args.workload)
    shapes = [(s.m, s.n) for s in wl.matrices]
    params = sum(m * n for m, n in shapes)
    print(f"[bench] workload {wl.key}: {len(shapes)} matrices, {params / 1e9:.3f} G params, "
          f"M {wl.m_dtype}, K={wl.K}, p={wl.power_iters}", flush=True)

    if args.calibrate_copy_mib > 0:
        nel = args.calibrate_copy_mib * (1 << 20) // 4
        src = torch.randn(nel, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print(f"[bench] calibration copy of {args.calibrate_copy_mib} MiB done", flush=True)
        del src, dst

    states = []
    for i, s in enumerate(wl.matrices):
        W0 = workloads.initial_weight(wl, i, dev)
        st = mo.new_state(s.m, s.n, wl.m_dtype, dev, W0=W0, rotated_momentum=args.rotated_momentum,
                          bases=not args.muon, bases16=args.bf16_bases)
        st["G"].copy_(workloads.gradient(wl, i, 1, dev))
        states.append(st)
    hp = mo.Hyper(wl.beta1, wl.beta2, wl.eps, wl.lr, wl.K, wl.power_iters, wl.capacity_bytes,
                  int(args.refresh_cap_gib * (1 << 30)), rotated_momentum=args.rotated_momentum,
                  bf16_rotation=args.bf16_rotation, muon=args.muon, ns_iters=args.ns_iters if args.muon else 0,
                  fp32_mfma=args.fp32_mfma, bf16_bases=args.bf16_bases)
    grp = mo.RotatedAdamGroup(states, hp)
    _, _, ngroups = mo.RotatedAdamGroup.plan(shapes, hp)
    # caller-owned state: W, G, M, v, U, V (and Mt)
    state_bytes = sum(t.numel() * t.element_size() for st in states for t in st.values())
    torch.cuda.synchronize()
    print(f"[bench] state ready, {ngroups} micro-groups, workspace {grp.ws_bytes / 1e9:.2f} GB", flush=True)

    for w in range(args.warmup):
        grp.step()
        torch.cuda.synchronize()
        print(f"[bench] warmup step {w + 1} done", flush=True)

    t_first = grp.t + 1
    refresh_steps = [t for t in range(t_first, t_first + args.steps)
                     if wl.K > 0 and (t - 1) % wl.K == 0]
    if not args.no_timing:
        grp.set_timing(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        grp.step()
        if (k + 1) % 5 == 0 or k + 1 == args.steps:
            print(f"[bench] timed step {k + 1}/{args.steps} enqueued", flush=True)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    phases = grp.read_timing() if not args.no_timing else {}
    group_ms = grp.read_group_timing() if not args.no_timing else []
    grp.set_timing(False)

    ms_per_step = 1e3 * elapsed / args.steps
    steps_per_s = args.steps / elapsed
    value = params * steps_per_s

    roofline = None
    extra = {}
    if phases and args.muon:
        ns_flops = sum(4.0 * min(m, n) ** 2 * max(m, n) for m, n in shapes) * args.ns_iters
        ms = phases["ortho"][0]
        achieved = ns_flops * args.steps / (ms * 1e-3) / 1e12 if ms > 0 else None
        mpeak = MI355X_FP32_MFMA_TFLOPS if args.fp32_mfma else X6_FP32_EQUIV_TFLOPS
        roofline = {
            "bound": "mfma", "achieved": achieved, "peak": mpeak, "unit": "TFLOP/s",
            "frac": achieved / mpeak if achieved else None, "traffic": None,
            "kernel": ("gemm_grouped_kernel" if args.fp32_mfma else "gemm_x6_kernel")
                      + " (Newton-Schulz X^T X and X (X^T X)"
                      + ("" if args.fp32_mfma else " on bf16 MFMAs, six piece products")
                      + "; the phase time includes the norm, scaling and combine kernels)",
            "launches": phases["ortho"][1], "avg_launch_ms": ms / max(phases["ortho"][1], 1),
            "flops_per_step": ns_flops,
        }
        extra["phase_ms_per_step"] = {k: v[0] / args.steps for k, v in phases.items() if v[1]}
        extra["phase_launches"] = {k: v[1] for k, v in phases.items() if v[1]}
    elif phases:
        no_flags = not (args.rotated_momentum or args.bf16_rotation or args.fp32_mfma)
        pf_all = phase_flops(shapes, m_dtype=wl.m_dtype, no_flags=no_flags)
        # the roofline is the dominant kernel's: the pieced bf16 products are reported beside it
        pf = {k: v for k, v in pf_all.items() if k != "rot_pieced"}
        flops = sum(pf.values()) * args.steps
        if args.rotated_momentum:   # recompute steps are the refreshes; the others carry m~
            carried = args.steps - len(refresh_steps)
            flops = sum(pf.values()) * len(refresh_steps) + sum(phase_flops(shapes, True).values()) * carried
        ms = sum(phases[k][0] for k in pf)
        launches = sum(phases[k][1] for k in pf)
        achieved = flops / (ms * 1e-3) / 1e12 if ms > 0 else None
        x6 = not (args.bf16_rotation or args.fp32_mfma)
        peak = (MI355X_BF16_MFMA_TFLOPS if args.bf16_rotation else
                X6_FP32_EQUIV_TFLOPS if x6 else MI355X_FP32_MFMA_TFLOPS)
        kernel = ("gemm16_kernel (bf16 rotation phases: (X V)^T, U^T S^T, (u V^T)^T, W -= lr U P^T)"
                  if args.bf16_rotation else
                  "gemm_x6_kernel (fp32 rotation phases on bf16 MFMAs, six piece products: U^T G, "
                  "(U^T G) V, the other product of M's chain, U u, W -= lr (.)V^T)" if "rot_pieced" in pf_all else
                  ("gemm_x6_kernel (rotation phases on bf16 MFMAs, six piece products: U^T[G|M], (.)V, "
                   "U u, W -= lr (.)V^T)" if x6 else
                   "gemm_grouped_kernel (rotation phases: U^T[G|M], (.)V, U u, W -= lr (.)V^T)"))
        roofline = {
            "bound": "mfma", "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
            "frac": achieved / peak if achieved else None,
            "traffic": None if args.bf16_rotation else traffic_per_launch(),
            "kernel": kernel,
            "launches": launches, "avg_launch_ms": ms / max(launches, 1),
            "flops_per_launch": flops / max(launches, 1),
            **({"peak_basis": "fp32-equivalent ceiling of six bf16 MFMA products per fp32 product "
                              "(2.5 PFLOP/s dense bf16 / 6)",
                "frac_of_fp32_mfma_peak": achieved / MI355X_FP32_MFMA_TFLOPS if achieved else None} if x6 else {}),
        }
        eb = elementwise_bytes(shapes, wl.m_dtype)
        extra["phase_ms_per_step"] = {k: v[0] / args.steps for k, v in phases.items() if v[1]}
        extra["phase_launches"] = {k: v[1] for k, v in phases.items() if v[1]}
        # per phase: the flops of the timed steps (carrying steps of the
        # rotated-momentum variant rotate G alone)
        pf_c = phase_flops(shapes, True)
        n_full = len(refresh_steps) if args.rotated_momentum else args.steps
        extra["phase_tflops"] = {k: ((pf[k] * n_full + pf_c[k] * (args.steps - n_full)) / (phases[k][0] * 1e-3) / 1e12
                                     if phases[k][0] else None) for k in pf}
        extra["elementwise_gbps"] = {k: (eb[k] * args.steps / (phases[k][0] * 1e-3) / 1e9 if phases[k][0] else None)
                                     for k in eb}
        if "rot_pieced" in pf_all and phases["rot_pieced"][0]:
            # fp32-equivalent algorithmic flops (2 m n max(m, n) per pieced matrix);
            # the bf16 MFMAs do three times as many
            ms_p = phases["rot_pieced"][0]
            eq = pf_all["rot_pieced"] * args.steps / (ms_p * 1e-3) / 1e12
            extra["pieced"] = {
                "kernel": "gemm16_kernel (U^T M or M V of a bf16 M, three exact bf16 pieces of the basis) "
                          "and the M^T copies it reads",
                "flops_per_step": pf_all["rot_pieced"], "ms_per_step": ms_p / args.steps,
                "fp32_equiv_tflops": eq, "bf16_mfma_tflops": 3 * eq,
                "bf16_frac": 3 * eq / MI355X_BF16_MFMA_TFLOPS,
                "rotations_tflops": (sum(pf_all.values()) * args.steps
                                     / ((ms + ms_p) * 1e-3) / 1e12),
            }
        if refresh_steps:
            extra["refresh_ms_each"] = phases["refresh"][0] / len(refresh_steps)
            # algorithmic flops of one refresh: p (8 m n r + (8/3)(m^3 + n^3)) per matrix
            rf = sum(wl.power_iters * (8.0 * m * n * min(m, n) + (8.0 / 3.0) * (m ** 3 + n ** 3)) for m, n in shapes)
            extra["refresh_tflops"] = rf / (extra["refresh_ms_each"] * 1e-3) / 1e12

    if group_ms:
        # per micro-group: its own launches (momentum, rotations, Adam, update,
        # pieced product) per step; the refresh runs over refresh batches and is
        # reported beside them
        _, group_of, _ = mo.RotatedAdamGroup.plan(shapes, hp)
        rows = []
        for k, ms_k in enumerate(group_ms):
            members = [i for i, gk in enumerate(group_of) if gk == k]
            p_k = sum(shapes[i][0] * shapes[i][1] for i in members)
            per_step = ms_k / args.steps
            rows.append({"group": k, "matrices": len(members), "params": p_k, "ms_per_step": per_step,
                         "steps_per_s": 1e3 / per_step if per_step > 0 else None,
                         "params_per_s": p_k * 1e3 / per_step if per_step > 0 else None})
        extra["micro_groups"] = rows
        if phases and phases.get("refresh", (0, 0))[0]:
            extra["refresh_ms_per_step"] = phases["refresh"][0] / args.steps

    if args.compare_single and roofline and roofline.get("flops_per_launch") and not (args.bf16_rotation or args.muon
                                                                                      or args.fp32_mfma):
        # one square fp32 product with the flops of an average rotation launch
        f = roofline["flops_per_launch"]
        side = max(256, int(round((f / 2.0) ** (1.0 / 3.0) / 256.0)) * 256)
        A = torch.randn(side, side, device=dev)
        B = torch.randn(side, side, device=dev)
        Cm = torch.empty(side, side, device=dev)
        s0 = mo.stream_ptr()
        mo.native.opt_gemm_x6(0, 0, side, side, side, 1.0, A.data_ptr(), 0, side, B.data_ptr(), 0, side, 0.0,
                              Cm.data_ptr(), side, s0)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(5):
            mo.native.opt_gemm_x6(0, 0, side, side, side, 1.0, A.data_ptr(), 0, side, B.data_ptr(), 0, side, 0.0,
                                  Cm.data_ptr(), side, s0)
        e1.record()
        torch.cuda.synchronize()
        ms1 = e0.elapsed_time(e1) / 5
        single = 2.0 * side ** 3 / (ms1 * 1e-3) / 1e12
        # a practical ceiling for comparison only (not part of the product):
        # torch's bf16 matmul (hipBLASLt) on the same shape, whose rate / 6 is
        # what six bf16 piece products per fp32 product could reach at that
        # library's efficiency
        Ab, Bb = A.to(torch.bfloat16), B.to(torch.bfloat16)
        torch.matmul(Ab, Bb)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(5):
            torch.matmul(Ab, Bb)
        e1.record()
        torch.cuda.synchronize()
        bf16_lib = 2.0 * side ** 3 / (e0.elapsed_time(e1) / 5 * 1e-3) / 1e12
        extra["single_product"] = {"shape": [side, side, side], "ms": ms1, "tflops": single,
                                   "grouped_tflops": roofline["achieved"],
                                   "grouped_over_single": roofline["achieved"] / single,
                                   "hipblaslt_bf16_tflops": bf16_lib,
                                   "grouped_over_hipblaslt_bf16_div6": roofline["achieved"] / (bf16_lib / 6)}
        del A, B, Cm, Ab, Bb

    cpu = None
    if args.cpu_sample_s > 0:
        print("[bench] timing the oracle on the host (cpu_baseline)", flush=True)
        cpu = cpu_baseline(wl, args.cpu_sample_s, args.ns_iters if args.muon else 0)

    out = {
        "metric": METRIC,
        "value": value,
        "unit": "params/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if args.bf16_rotation else "f32",
        "data": "synthetic",
        "config": {"workload": wl.key, "matrices": len(shapes), "params": params,
                   "momentum_dtype": wl.m_dtype, "K": wl.K, "power_iters": wl.power_iters,
                   "micro_groups": ngroups, "refresh_steps_timed": refresh_steps,
                   "workspace_bytes": grp.ws_bytes,
                   "state_bytes": state_bytes,
                   "rotated_momentum": bool(args.rotated_momentum),
                   "bf16_rotation": bool(args.bf16_rotation), "bf16_bases": bool(args.bf16_bases),
                   "muon": bool(args.muon),
                   "fp32_mfma": bool(args.fp32_mfma),
                   # how the fp32 products execute: six bf16 MFMA piece products each (fp32 accuracy),
                   # or fp32 MFMAs
                   "fp32_products": ("fp32 MFMA" if args.fp32_mfma
                                     else "bf16 MFMA, three-piece split, six piece products"),
                   **({"ns_iters": args.ns_iters} if args.muon else {})},
        "steps_per_s": steps_per_s,
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    out.update(extra)
    grp.close()
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
