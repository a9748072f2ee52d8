"""Host-side tests of the C ABI: the library loads, exports every entry point
include/matopt.h declares, plans micro-groups as specified, and rejects bad
arguments before touching the device (no GPU needed)."""

import ctypes as C
import os
import re

import pytest

import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def N():
    from matrix_optimizer_step_02_amd import native
    if not os.path.exists(native.LIB_PATH):
        pytest.skip("libmatopt.so not built (run __graft_entry__.build())")
    native.load()
    return native


def header_functions():
    txt = open(os.path.join(ROOT, "include", "matopt.h")).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(opt_[a-z0-9_]+)\s*\(", txt)))


def test_every_declared_symbol_is_exported(N):
    names = header_functions()
    assert len(names) >= 15
    lib = N.load()
    for name in names:
        assert hasattr(lib, name), name
    assert set(names) == set(N.EXPORTED)


def hp(N, **kw):
    base = dict(beta1=0.9, beta2=0.999, eps=1e-8, lr=1e-3, K=10, power_iters=1, capacity_bytes=0, refresh_capacity_bytes=0, flags=0,
                ns_iters=0)
    base.update(kw)
    return N.opt_hparams(**base)


def descs(N, shapes, dtype=0, ptrs=False):
    out = []
    base = 1 << 40
    for i, (m, n) in enumerate(shapes):
        if ptrs:
            p = [base + (i * 6 + k) * (1 << 32) for k in range(6)]
            out.append(N.opt_matrix_desc(m, n, p[0], p[1], p[2], dtype, p[3], p[4], p[5]))
        else:
            out.append(N.opt_matrix_desc(m, n, 0, 0, 0, dtype, 0, 0, 0))
    return out


def ref_plan(shapes, cap=1 << 29):
    """Independent statement of the planner: stable LPT by m*n*(m+n), next-fit
    groups of total 4*m*n within the cap."""
    order = sorted(range(len(shapes)), key=lambda i: -shapes[i][0] * shapes[i][1] * (shapes[i][0] + shapes[i][1]))
    groups, used = [], None
    for i in order:
        b = 4 * shapes[i][0] * shapes[i][1]
        if used is None or used + b > cap:
            groups.append([])
            used = 0
        groups[-1].append(i)
        used += b
    gof = [0] * len(shapes)
    for g, mem in enumerate(groups):
        for i in mem:
            gof[i] = g
    return order, gof, len(groups)


@pytest.mark.parametrize("key", ["tiny", "layer", "qwen3_1p7b", "microgroup_512mib", "qwen3_8b_half"])
def test_plan_matches_reference(N, key):
    wl = workloads.get(key)
    shapes = [(s.m, s.n) for s in wl.matrices]
    got = N.opt_plan(descs(N, shapes), hp(N))
    assert got == ref_plan(shapes)


def test_plan_known_counts(N):
    q = [(s.m, s.n) for s in workloads.get("qwen3_1p7b").matrices]
    assert N.opt_plan(descs(N, q), hp(N))[2] == 11
    mg = [(s.m, s.n) for s in workloads.get("microgroup_512mib").matrices]
    assert sum(4 * m * n for m, n in mg) == 1 << 29        # the draw fills the cap exactly
    assert N.opt_plan(descs(N, mg), hp(N))[2] == 1


def test_plan_lpt_ties_keep_input_order(N):
    shapes = [(8, 8), (16, 4), (4, 16), (8, 8), (32, 32)]
    order, _, _ = N.opt_plan(descs(N, shapes), hp(N))
    assert order == [4, 0, 3, 1, 2] or order == [4, 1, 2, 0, 3]
    costs = [shapes[i][0] * shapes[i][1] * sum(shapes[i]) for i in order]
    assert costs == sorted(costs, reverse=True)
    assert order == ref_plan(shapes)[0]


def test_plan_custom_capacity(N):
    shapes = [(64, 64)] * 10
    order, gof, ng = N.opt_plan(descs(N, shapes), hp(N, capacity_bytes=3 * 4 * 64 * 64))
    assert ng == 4 and gof == [0, 0, 0, 1, 1, 1, 2, 2, 2, 3]


def err(N, fn, *a):
    with pytest.raises(N.MatoptError) as e:
        fn(*a)
    return e.value.status


def test_rejects_bad_hyperparameters(N):
    d = descs(N, [(8, 8)])
    for kw in (dict(beta1=1.0), dict(beta1=-0.1), dict(beta2=1.0), dict(eps=0.0), dict(eps=float("inf")),
               dict(lr=float("nan")), dict(K=-1), dict(power_iters=0), dict(flags=4), dict(flags=1 << 31)):
        assert err(N, N.opt_group_workspace_size, d, hp(N, **kw)) == N.OPT_EINVAL, kw


def test_flag_combinations(N):
    d = descs(N, [(8, 8)])
    N.opt_group_workspace_size(d, hp(N, flags=N.OPT_FLAG_BF16_ROTATION))
    N.opt_group_workspace_size(d, hp(N, flags=N.OPT_FLAG_BF16_ROTATION | N.OPT_FLAG_ROTATED_MOMENTUM))


def test_muon_flag_checks(N):
    d = descs(N, [(8, 8)])
    N.opt_group_workspace_size(d, hp(N, flags=N.OPT_FLAG_MUON, ns_iters=2))
    N.opt_group_workspace_size(d, hp(N, flags=N.OPT_FLAG_MUON | N.OPT_FLAG_FP32_MFMA, ns_iters=2))
    assert err(N, N.opt_group_workspace_size, d, hp(N, flags=N.OPT_FLAG_MUON)) == N.OPT_EINVAL    # ns_iters 0
    for other in (N.OPT_FLAG_BF16_ROTATION, N.OPT_FLAG_ROTATED_MOMENTUM):
        assert err(N, N.opt_group_workspace_size, d, hp(N, flags=N.OPT_FLAG_MUON | other, ns_iters=2)) == \
            N.OPT_EUNSUPPORTED
    # v, U, V may be NULL with the flag, not without it
    d = descs(N, [(8, 8)], ptrs=True)
    d[0].v = d[0].U = d[0].V = 0
    need = N.opt_group_workspace_size(d, hp(N, flags=N.OPT_FLAG_MUON, ns_iters=2))
    assert err(N, N.opt_group_create, d, hp(N), 1 << 44, 1 << 30, 0) == N.OPT_EINVAL
    assert need < 1 << 20


def _parts(N, d, h):
    p = N.opt_group_workspace_parts(d, h)
    assert N.opt_group_workspace_size(d, h) == p["tables"] + max(p["copies"] + p["scratch"], p["refresh"])
    return p


def test_workspace_holds_the_copies_of_the_bases(N):
    """The fp32 rotations keep an fp32 U^T (4 m^2 bytes, 256-byte aligned)
    per matrix; the bf16 variant instead keeps bf16 U, U^T, V, V^T (rows
    padded to multiples of 8 elements) and a larger scratch; Muon keeps
    neither. The carried rotated momentum adds the work lists of its two
    kinds of step (its m~ is caller-owned). The size is the tables plus the
    larger of (copies + scratch) and the largest refresh batch."""
    shapes = [(130, 67), (64, 64), (24, 40)]
    d = descs(N, shapes)
    base = _parts(N, d, hp(N))
    var = _parts(N, d, hp(N, flags=N.OPT_FLAG_BF16_ROTATION))
    rm = _parts(N, d, hp(N, flags=N.OPT_FLAG_ROTATED_MOMENTUM))
    mu = _parts(N, d, hp(N, flags=N.OPT_FLAG_MUON, ns_iters=2))
    r8 = lambda x: (x + 7) // 8 * 8
    a256 = lambda x: (x + 255) // 256 * 256
    ut = sum(a256(4 * m * m) for m, _ in shapes)
    bases = sum(a256(2 * m * r8(m)) * 2 + a256(2 * n * r8(n)) * 2 for m, n in shapes)
    assert base["copies"] == ut and rm["copies"] == ut
    assert var["copies"] == bases
    assert mu["copies"] == 0 and mu["refresh"] == 0
    assert base["scratch"] >= sum(16 * m * n for m, n in shapes[:1])
    assert var["scratch"] > base["scratch"]
    assert rm["scratch"] == base["scratch"] and base["tables"] < rm["tables"] < base["tables"] + 64 * 1024
    # the refresh buffers do not depend on how the step rotates
    assert base["refresh"] == rm["refresh"] == var["refresh"] > 0


def test_refresh_buffers_overlay_the_copies(N):
    """The default refresh cap is the larger of 4 GiB and the copies plus the
    scratch, so a refresh batch never makes the workspace larger than that
    unless one matrix alone needs more; an explicit cap splits the batches
    (a matrix above it forms a batch alone)."""
    shapes = [(4096, 4096), (4096, 1024), (1024, 4096), (2048, 2048)]
    d = descs(N, shapes, dtype=N.OPT_BF16)
    p = _parts(N, d, hp(N))
    assert p["refresh"] <= max(4 << 30, p["copies"] + p["scratch"])
    one = _parts(N, d, hp(N, refresh_capacity_bytes=1))
    assert one["refresh"] < p["refresh"]
    assert (one["tables"], one["copies"], one["scratch"]) != (0, 0, 0)
    assert one["copies"] == p["copies"] and one["scratch"] == p["scratch"]


def test_default_refresh_cap_keeps_the_qwen3_sets_in_one_batch(N):
    """The default refresh cap (the largest of 4 GiB, the copies and scratch,
    and the state) gives the Qwen3-1.7B set and the Qwen3-8B half one refresh
    batch each (the same largest batch as an unbounded cap), with a
    workspace below the state it serves."""
    for key in ("qwen3_1p7b", "qwen3_8b_half"):
        wl = workloads.get(key)
        dt = N.OPT_BF16 if wl.m_dtype == "bf16" else N.OPT_F32
        d = descs(N, [(s.m, s.n) for s in wl.matrices], dtype=dt)
        default = _parts(N, d, hp(N, K=wl.K))
        unbounded = _parts(N, d, hp(N, K=wl.K, refresh_capacity_bytes=1 << 50))
        assert default["refresh"] == unbounded["refresh"]
        state = sum(s.m * s.n * (12 + (2 if wl.m_dtype == "bf16" else 4)) + 4 * (s.m ** 2 + s.n ** 2)
                    for s in wl.matrices)
        assert N.opt_group_workspace_size(d, hp(N, K=wl.K)) <= state


def test_workspace_holds_the_pieces_of_the_momentum_bases(N):
    """A bf16 M with both sides multiples of 8 gets the three bf16 pieces of
    U^T (m > n) or V^T (m <= n), 6 d^2 bytes (256-byte aligned), beside the
    fp32 U^T copy; fp32 M, ragged sides, and the flag that keeps the
    rotations on fp32 MFMAs add nothing."""
    shapes = [(200, 72), (72, 264), (136, 136), (130, 67), (8, 8)]
    a256 = lambda x: (x + 255) // 256 * 256
    bf = descs(N, shapes, dtype=N.OPT_BF16)
    pieced = _parts(N, bf, hp(N))
    plain = _parts(N, bf, hp(N, flags=N.OPT_FLAG_FP32_MFMA))
    f32 = descs(N, shapes)
    pieces = sum(a256(6 * max(m, n) ** 2) for m, n in shapes if m % 8 == 0 and n % 8 == 0)
    assert pieced["copies"] - plain["copies"] == pieces
    assert 0 <= pieced["tables"] - plain["tables"] < 16 * 1024    # the work lists of the new launches
    assert N.opt_group_workspace_parts(f32, hp(N)) == N.opt_group_workspace_parts(f32, hp(N, flags=N.OPT_FLAG_FP32_MFMA))
    for other in (N.OPT_FLAG_ROTATED_MOMENTUM, N.OPT_FLAG_BF16_ROTATION):
        assert N.opt_group_workspace_parts(bf, hp(N, flags=other)) == \
            N.opt_group_workspace_parts(bf, hp(N, flags=other | N.OPT_FLAG_FP32_MFMA))


def test_rejects_bad_shapes_and_dtypes(N):
    assert err(N, N.opt_group_workspace_size, descs(N, [(0, 4)]), hp(N)) == N.OPT_EINVAL
    assert err(N, N.opt_group_workspace_size, descs(N, [(4, -1)]), hp(N)) == N.OPT_EINVAL
    assert err(N, N.opt_group_workspace_size, descs(N, [(N.OPT_MAX_DIM + 1, 4)]), hp(N)) == N.OPT_EUNSUPPORTED
    assert err(N, N.opt_group_workspace_size, descs(N, [(4, 4)], dtype=7), hp(N)) == N.OPT_EUNSUPPORTED
    # a matrix bigger than the capacity cannot be split
    assert err(N, N.opt_group_workspace_size, descs(N, [(4096, 4096)]), hp(N, capacity_bytes=1 << 20)) == N.OPT_EINVAL
    assert err(N, N.opt_group_workspace_size, [], hp(N)) == N.OPT_EINVAL


def test_create_rejects_before_any_device_call(N):
    h = hp(N)
    ws = 1 << 44
    assert err(N, N.opt_group_create, descs(N, [(8, 8)]), h, ws, 1 << 30, 0) == N.OPT_EINVAL  # null tensors
    d = descs(N, [(8, 8), (8, 8)], ptrs=True)
    d[1].W = d[0].W + 16  # overlaps matrix 0's W
    assert err(N, N.opt_group_create, d, h, ws, 1 << 30, 0) == N.OPT_EINVAL
    d = descs(N, [(8, 8)], ptrs=True)
    need = N.opt_group_workspace_size(d, h)
    assert err(N, N.opt_group_create, d, h, ws, need - 1, 0) == N.OPT_ENOWS
    assert err(N, N.opt_group_create, d, h, 0, need, 0) == N.OPT_EINVAL
    assert err(N, N.opt_group_create, d, h, ws + 8, need, 0) == N.OPT_EINVAL      # not 256-aligned
    d[0].W = ws + 256                                                            # tensor inside workspace
    assert err(N, N.opt_group_create, d, h, ws, need, 0) == N.OPT_EINVAL
    d = descs(N, [(8, 8)], ptrs=True)
    d[0].W = ws - 64                                  # starts below the workspace, its tail runs into it
    assert err(N, N.opt_group_create, d, h, ws, need, 0) == N.OPT_EINVAL
    assert "overlaps the workspace" in N.opt_last_error()
    d = descs(N, [(8, 8)], ptrs=True)
    hr = hp(N, flags=N.OPT_FLAG_ROTATED_MOMENTUM)
    need_r = N.opt_group_workspace_size(d, hr)       # no pointer is read: Mt may be unset here
    d[0].Mt = (1 << 40) + 7 * (1 << 32)
    assert N.opt_group_workspace_size(d, hr) == need_r
    d[0].Mt = ws + need_r - 4                         # the carried momentum starts in the last word
    assert err(N, N.opt_group_create, d, hr, ws, need_r, 0) == N.OPT_EINVAL
    assert "Mt overlaps the workspace" in N.opt_last_error()
    d = descs(N, [(8, 8)], ptrs=True)
    d[0].M = d[0].M + 1                                                          # misaligned
    assert err(N, N.opt_group_create, d, h, ws, need, 0) == N.OPT_EINVAL
    # the rotated momentum needs Mt exactly when its flag is set, not overlapping
    d = descs(N, [(8, 8)], ptrs=True)
    hr = hp(N, flags=N.OPT_FLAG_ROTATED_MOMENTUM)
    assert err(N, N.opt_group_create, d, hr, ws, need, 0) == N.OPT_EINVAL         # flag without Mt
    d[0].Mt = (1 << 40) + 7 * (1 << 32)
    assert err(N, N.opt_group_create, d, h, ws, need, 0) == N.OPT_EINVAL          # Mt without flag
    d[0].Mt = d[0].v + 64
    assert err(N, N.opt_group_create, d, hr, ws, need, 0) == N.OPT_EINVAL         # Mt overlaps v


def test_null_group_and_bad_building_block_args(N):
    assert err(N, N.opt_group_step, 0, 0) == N.OPT_EINVAL
    assert err(N, N.opt_group_get_step, 0) == N.OPT_EINVAL
    assert err(N, N.opt_group_set_step, 0, 3) == N.OPT_EINVAL
    assert err(N, N.opt_group_refresh_basis, 0, 1, 0) == N.OPT_EINVAL
    N.opt_group_destroy(0)
    assert err(N, N.opt_gemm, 0, 0, -1, 4, 4, 1.0, 1, 0, 4, 1, 0, 4, 0.0, 1, 4, 0) == N.OPT_EINVAL
    assert err(N, N.opt_gemm, 0, 0, 4, 4, 4, 1.0, 1, 3, 4, 1, 0, 4, 0.0, 1, 4, 0) == N.OPT_EUNSUPPORTED
    assert err(N, N.opt_gemm, 0, 0, 4, 4, 8, 1.0, 1, 0, 4, 1, 0, 4, 0.0, 1, 4, 0) == N.OPT_EINVAL  # lda < K
    N.opt_gemm(0, 0, 0, 4, 4, 1.0, 0, 0, 4, 0, 0, 4, 0.0, 0, 4, 0)              # empty: no-op
    # bf16 GEMM: K, lda, ldb multiples of 8, A and B 16-byte aligned, a bf16 C without beta
    g16 = dict(M=4, N=4, K=8, alpha=1.0, A=1 << 40, lda=8, B=1 << 41, ldb=8, beta=0.0, Cp=1 << 42, c_dtype=0,
               ldc=4, stream_ptr=0)
    for kw, st in ((dict(K=7), N.OPT_EINVAL), (dict(lda=12), N.OPT_EINVAL), (dict(A=(1 << 40) + 8), N.OPT_EINVAL),
                   (dict(c_dtype=1, beta=1.0), N.OPT_EINVAL), (dict(c_dtype=5), N.OPT_EUNSUPPORTED),
                   (dict(ldc=3), N.OPT_EINVAL), (dict(M=-1), N.OPT_EINVAL), (dict(lda=4, K=8), N.OPT_EINVAL)):
        assert err(N, lambda: N.opt_gemm_bf16(**dict(g16, **kw))) == st, kw
    N.opt_gemm_bf16(**dict(g16, M=0))                                           # empty: no-op
    assert err(N, N.opt_orthonormalize_workspace_size, 0) == N.OPT_EINVAL
    assert err(N, N.opt_orthonormalize_workspace_size, N.OPT_MAX_DIM + 1) == N.OPT_EUNSUPPORTED
    assert N.opt_orthonormalize_workspace_size(100) > 0


def test_workspace_is_max_over_groups(N):
    """Scratch is sized for the largest micro-group (or refresh batch), not
    the sum; the fp32 U^T copies (4 MiB per matrix here) are per matrix."""
    h = hp(N, refresh_capacity_bytes=1 << 30)
    ut = 4 * 1024 * 1024
    one_group = N.opt_group_workspace_size(descs(N, [(1024, 1024)] * 128), h) - 128 * ut  # 128 x 4 MiB = cap
    two_groups = N.opt_group_workspace_size(descs(N, [(1024, 1024)] * 200), h) - 200 * ut
    assert N.opt_plan(descs(N, [(1024, 1024)] * 200), h)[2] == 2
    assert one_group <= two_groups < 1.05 * one_group
    assert one_group >= 128 * 4 * 4 * 1024 * 1024          # four m x n rotation buffers per matrix


def test_refresh_batches_follow_their_cap(N):
    d = descs(N, [(2048, 2048)] * 64)
    small = N.opt_group_workspace_size(d, hp(N, refresh_capacity_bytes=1 << 28))
    large = N.opt_group_workspace_size(d, hp(N, refresh_capacity_bytes=1 << 36))
    assert small < large
    assert large >= 64 * 2 * 4 * 2048 * 2048               # every QR input of one batch


def test_bench_selects_rotation_dispatches_from_non_refresh_steps():
    """The counter summary takes only grouped GEMMs of steps without a QR
    kernel: the refresh uses the same GEMM instantiations."""
    import bench
    name = ("void matopt::(anonymous namespace)::gemm_grouped_kernel<matopt::(anonymous namespace)::"
            "Cfg<2, 2, 4, 2, 16>, false, {}, false, {}>(matopt::(anonymous namespace)::GemmArgs)")
    gemm, bf16_b, bt = name.format("false", "false"), name.format("false", "true"), name.format("true", "false")
    x6 = ("void matopt::(anonymous namespace)::gemm_x6_kernel<matopt::(anonymous namespace)::Cfg<2, 2, 4, 2, 16>, "
          "false, false, false>(matopt::(anonymous namespace)::GemmArgs)")
    seq = ["copyBuffer", "momentum_kernel", "momentum_kernel", gemm, "qr_panel_kernel", gemm, gemm,
           "rotated_adam_kernel", gemm, "momentum_kernel", "momentum_kernel", gemm, bf16_b, gemm,
           "rotated_adam_kernel", x6, bt, "gemm16_kernel<Cfg16<2, 2, 4, 4, 64, 2>, false>(Gemm16Args)"]
    rows = [{"Dispatch_Id": str(i + 1), "Kernel_Name": k} for i, k in enumerate(seq)]
    picked = bench.rotation_dispatches(list(reversed(rows)))
    assert [int(r["Dispatch_Id"]) for r in picked] == [12, 13, 14, 16, 17]


def test_bench_flop_accounting_covers_the_rotations_once():
    """Whatever the path, the per-phase flops of a full step add up to the
    rotations' 6 m n (m + n); without flags a bf16 M with sides multiples of
    8 moves 2 m n max(m, n) to the pieced phase (U^T M when m > n, M V
    otherwise), and the carrying step of the rotated momentum rotates G
    alone (4 m n (m + n))."""
    import bench
    shapes = [(2048, 2048), (2048, 1024), (2048, 6144), (6144, 2048), (130, 67), (8, 16)]
    total = bench.rotation_flops(shapes)
    for m_dtype in ("f32", "bf16"):
        for no_flags in (False, True):
            pf = bench.phase_flops(shapes, m_dtype=m_dtype, no_flags=no_flags)
            assert abs(sum(pf.values()) - total) <= 1e-9 * total
            pieced = sum(2.0 * m * n * max(m, n) for m, n in shapes
                         if no_flags and m_dtype == "bf16" and m % 8 == 0 and n % 8 == 0)
            assert pf.get("rot_pieced", 0.0) == pieced
    carry = bench.phase_flops(shapes, carry=True)
    assert abs(sum(carry.values()) - sum(4.0 * m * n * (m + n) for m, n in shapes)) <= 1e-9 * total
