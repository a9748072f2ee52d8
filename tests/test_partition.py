"""Cross-rank planners: the oracle against closed forms, invariants and brute
force, then the library's C planners against the oracle, result for result.

Both planners are integer decisions taken from float64 sums in a fixed order,
so the library must reproduce the oracle exactly (owners, cut points, groups,
host ranks) and its loads bit for bit.
"""

import itertools
import math
import random

import pytest

import workloads
from oracle import partition as P


def _native():
    import matrix_optimizer_step_02_amd as mo
    return mo.native


def _check_geometry(owner, bucket_begin, R):
    """Every parameter owned; along each bucket the owners never decrease
    (rank r holds one consecutive range, ranks in order)."""
    assert all(0 <= o < R for o in owner)
    for b in range(len(bucket_begin) - 1):
        seg = owner[bucket_begin[b]:bucket_begin[b + 1]]
        assert all(x <= y for x, y in zip(seg, seg[1:]))


# ---------------------------------------------------------------- oracle pins

def test_single_bucket_of_equal_costs_splits_evenly():
    """One bucket of R*q unit costs: every alpha gives each rank q
    consecutive parameters (the targets are multiples of q exactly)."""
    for R, q in [(1, 5), (2, 3), (4, 4), (8, 2)]:
        for alpha in (0.0, 0.5, 1.0):
            owner, loads = P.alpha_balanced_partition([1.0] * (R * q), [0, R * q], R, alpha)
            assert owner == [r for r in range(R) for _ in range(q)]
            assert loads == [float(q)] * R


def test_alpha_zero_ignores_earlier_loads():
    """alpha = 0: the shares are 1/R whatever the loads, so a bucket is cut
    the same way when placed alone or after others."""
    costs_a = [5.0, 1.0, 1.0, 1.0, 1.0, 1.0]
    costs_b = [1.0] * 4
    owner_ab, _ = P.alpha_balanced_partition(costs_a + costs_b, [0, 6, 10], 2, 0.0)
    owner_b, _ = P.alpha_balanced_partition(costs_b, [0, 4], 2, 0.0)
    assert owner_ab[6:] == owner_b == [0, 0, 1, 1]
    assert P.bucket_shares([7.0, 0.0, 3.0], 4.0, 0.0) == [1 / 3] * 3


def _printed_shares_hold():
    """The Canzona page, section 3.2.1: a rank's deficit is its gap below the
    mean of the current loads, sum(L) / R; at alpha = 1 the shares are the
    deficits normalised. Loads [4, 2, 0, 3] have mean 9/4, deficits
    [0, 1/4, 9/4, 0] (sum 5/2), so a bucket of 11 is shared [0, 0.1, 0.9, 0]
    whatever its cost; at alpha = 1/2 the even split enters half-way:
    [1/8, 7/40, 23/40, 1/8]. Cut into 44 parameters of 1/4, the targets
    0, 1.1, 11 snap to boundaries 0, 4, 44."""
    loads = [4.0, 2.0, 0.0, 3.0]
    if P.bucket_shares(loads, 11.0, 1.0) != pytest.approx([0.0, 0.1, 0.9, 0.0], rel=1e-15, abs=1e-300):
        return False
    if P.bucket_shares(loads, 11.0, 0.5) != pytest.approx([1 / 8, 7 / 40, 23 / 40, 1 / 8], rel=1e-15):
        return False
    cuts = P.atomic_cuts([0.25] * 44, P.bucket_shares(loads, 11.0, 1.0))
    return cuts == [0, 0, 4, 44, 44]


def test_alpha_one_shares_follow_the_printed_deficits():
    assert _printed_shares_hold()


def test_shares_closed_forms():
    """No rank below the mean (the first bucket, equal loads): the even split
    for every alpha. Two ranks with loads a > b: at alpha the trailing rank
    gets (1 - alpha)/2 + alpha, the leading one (1 - alpha)/2."""
    for alpha in (0.0, 0.3, 1.0):
        assert P.bucket_shares([0.0] * 5, 7.0, alpha) == pytest.approx([0.2] * 5, rel=1e-15)
        assert P.bucket_shares([3.0] * 4, 1.0, alpha) == pytest.approx([0.25] * 4, rel=1e-15)
        assert P.bucket_shares([5.0, 2.0], 9.0, alpha) == pytest.approx(
            [(1 - alpha) / 2, (1 - alpha) / 2 + alpha], rel=1e-15, abs=1e-300)


def test_alpha_one_gives_nothing_to_ranks_at_or_above_the_mean():
    """At alpha = 1 a bucket is placed only on ranks whose load was below the
    mean of the loads before it (unless no rank trailed); over random cases."""
    rng = random.Random(3)
    for case in range(200):
        R = rng.randint(2, 9)
        loads = [rng.choice([0.0, 1.0, 2.0, rng.uniform(0, 5)]) for _ in range(R)]
        costs = [rng.uniform(0.1, 1.0) for _ in range(rng.randint(1, 30))]
        shares = P.bucket_shares(loads, sum(costs), 1.0)
        cuts = P.atomic_cuts(costs, shares)
        mean = sum(loads) / R
        if any(x < mean for x in loads):
            for r in range(R):
                if loads[r] >= mean:
                    assert shares[r] == 0.0 and cuts[r + 1] == cuts[r]


def test_planted_mean_after_placement_is_caught(monkeypatch):
    """Deficits against the mean after the bucket, (sum(L) + W) / R (a reading
    that water-fills every trailing rank), give [1/11, 3/11, 5/11, 2/11] on
    the printed case: the pin fails."""
    def shares_after(loads, W, alpha):
        R = len(loads)
        mean = (sum(loads) + W) / R
        d = [max(0.0, mean - x) for x in loads]
        s = sum(d)
        fill = [x / s for x in d] if s > 0 else [1.0 / R] * R
        return [(1 - alpha) / R + alpha * f for f in fill]
    monkeypatch.setattr(P, "bucket_shares", shares_after)
    assert not _printed_shares_hold()


def test_planted_unsorted_buckets_are_caught(monkeypatch):
    """Placing buckets in input order instead of largest first changes the
    Qwen3-1.7B partition at 8 ranks (LPT order is part of the method)."""
    mats, bb = workloads.planning_set("qwen3_1p7b")
    # later layers slightly costlier, so that input order is the reverse of LPT order
    costs = [P.matrix_step_cost(s.m, s.n, 10, 1) * (1.0 + 0.01 * s.layer) for s in mats]
    ref, _ = P.alpha_balanced_partition(costs, bb, 8, 1.0)
    real_sorted = sorted
    monkeypatch.setattr("builtins.sorted", lambda it, key=None, reverse=False: list(it))
    try:
        planted, _ = P.alpha_balanced_partition(costs, bb, 8, 1.0)
    finally:
        monkeypatch.setattr("builtins.sorted", real_sorted)
    assert planted != ref


def test_cuts_snap_to_nearest_boundary_with_ties_to_the_shorter_prefix():
    # prefixes 0, 3, 4, 10; target 5 (half of 10): 4 is nearest
    assert P.atomic_cuts([3.0, 1.0, 6.0], [0.5, 0.5]) == [0, 2, 3]
    # a single parameter: target 1.5 between 0 and 3, a tie -> empty first range
    assert P.atomic_cuts([3.0], [0.5, 0.5]) == [0, 0, 1]
    # zero-cost parameters and an empty bucket
    assert P.atomic_cuts([0.0, 0.0], [0.5, 0.5]) == [0, 0, 2]
    assert P.atomic_cuts([], [0.25] * 4) == [0, 0, 0, 0, 0]


def test_random_partitions_keep_geometry_and_loads():
    rng = random.Random(11)
    for case in range(40):
        R = rng.randint(1, 9)
        nb = rng.randint(1, 8)
        costs, bb = [], [0]
        for b in range(nb):
            k = rng.randint(0, 9)
            costs += [float(rng.choice([0, 1, 2, 3, 7, 7, 13])) for _ in range(k)]
            bb.append(len(costs))
        alpha = rng.choice([0.0, 0.3, 1.0])
        owner, loads = P.alpha_balanced_partition(costs, bb, R, alpha)
        _check_geometry(owner, bb, R)
        for r in range(R):
            assert loads[r] == pytest.approx(sum(c for c, o in zip(costs, owner) if o == r))


def _graham_bound_ok(costs, hosts, R):
    """LPT list scheduling (the min-heap) has makespan <= (4/3 - 1/(3R)) OPT
    (Graham, 1969); OPT by brute force over every assignment."""
    span = max(sum(c for c, h in zip(costs, hosts) if h == r) for r in range(R))
    best = math.inf
    for assign in itertools.product(range(R), repeat=len(costs)):
        best = min(best, max(sum(c for c, a in zip(costs, assign) if a == r) for r in range(R)))
    return span <= (4 / 3 - 1 / (3 * R)) * best + 1e-12


def test_host_ranks_are_lpt_within_graham_bound():
    rng = random.Random(5)
    for case in range(25):
        n = rng.randint(1, 7)
        R = rng.randint(1, 3)
        costs = [float(rng.randint(1, 20)) for _ in range(n)]
        nbytes = [1] * n
        order, group_of, host_of, ng = P.micro_groups_host_ranks(costs, nbytes, R, 1 << 40)
        assert ng == 1
        assert [costs[i] for i in order] == sorted(costs, reverse=True)
        assert _graham_bound_ok(costs, host_of, R)


def test_micro_groups_respect_capacity_in_lpt_order():
    costs = [9.0, 8.0, 7.0, 6.0, 5.0, 4.0]
    nbytes = [4, 4, 4, 12, 1, 1]
    order, group_of, host_of, ng = P.micro_groups_host_ranks(costs, nbytes, 2, 8)
    # LPT order 0..5; groups {0,1}, {2}, {3} (alone: larger than the cap), {4,5}
    assert order == [0, 1, 2, 3, 4, 5]
    assert group_of == [0, 0, 1, 2, 3, 3]
    assert host_of == [0, 1, 0, 0, 0, 1]
    assert ng == 4


def test_capacity_one_group_per_parameter_and_single_rank():
    order, group_of, host_of, ng = P.micro_groups_host_ranks([1.0, 2.0, 3.0], [5, 5, 5], 1, 5)
    assert group_of == [2, 1, 0] and host_of == [0, 0, 0] and ng == 3


# ------------------------------------------------------------ library vs oracle

def _random_case(rng):
    R = rng.randint(1, 12)
    nb = rng.randint(0, 10)
    costs, bb = [], [0]
    for b in range(nb):
        k = rng.randint(0, 12)
        kind = rng.random()
        for _ in range(k):
            if kind < 0.3:
                costs.append(float(rng.choice([0, 1, 1, 2, 5])))      # many exact ties
            else:
                costs.append(rng.lognormvariate(0, 2))
        bb.append(len(costs))
    return costs, bb, R, rng.choice([0.0, 0.25, 0.5, 0.8, 1.0])


def test_library_partition_matches_oracle_on_random_cases():
    N = _native()
    rng = random.Random(2024)
    for case in range(300):
        costs, bb, R, alpha = _random_case(rng)
        ref_owner, ref_loads = P.alpha_balanced_partition(costs, bb, R, alpha)
        owner, loads = N.opt_partition_dp(costs, bb, R, alpha)
        assert owner == ref_owner, (case, R, alpha)
        assert loads == ref_loads, (case, R, alpha)


def test_library_host_ranks_match_oracle_on_random_cases():
    N = _native()
    rng = random.Random(77)
    for case in range(300):
        n = rng.randint(0, 40)
        R = rng.randint(1, 9)
        costs = [float(rng.choice([0, 1, 2, 3, 3, 8])) if rng.random() < 0.4 else rng.lognormvariate(0, 1.5)
                 for _ in range(n)]
        nbytes = [rng.choice([0, 1, 3, 8, 20]) for _ in range(n)]
        cap = rng.choice([1, 8, 20, 64])
        ref = P.micro_groups_host_ranks(costs, nbytes, R, cap)
        got = N.opt_plan_host_ranks(costs, nbytes, R, cap)
        assert tuple(got) == tuple(ref), case


@pytest.mark.parametrize("model", sorted(workloads.PLANNING_MODELS))
def test_library_planners_match_oracle_on_qwen3_models(model):
    N = _native()
    mats, bb = workloads.planning_set(model)
    K = 10 if model == "qwen3_1p7b" else 5
    costs = [P.matrix_step_cost(s.m, s.n, K, 1) for s in mats]
    nbytes = [4 * s.m * s.n for s in mats]
    for R in (8, 16, 32, 64, 128, 256):
        for alpha in (0.0, 1.0):
            assert N.opt_partition_dp(costs, bb, R, alpha) == P.alpha_balanced_partition(costs, bb, R, alpha)
    for R in (1, 2, 4, 8):
        assert tuple(N.opt_plan_host_ranks(costs, nbytes, R, 1 << 29)) == \
            tuple(P.micro_groups_host_ranks(costs, nbytes, R, 1 << 29))


def test_library_planner_argument_errors():
    N = _native()
    with pytest.raises(N.MatoptError):
        N.opt_partition_dp([1.0], [0, 1], 0, 1.0)
    with pytest.raises(N.MatoptError):
        N.opt_partition_dp([1.0], [0, 1], 2, 1.5)
    with pytest.raises(N.MatoptError):
        N.opt_partition_dp([-1.0], [0, 1], 2, 1.0)
    with pytest.raises(N.MatoptError):
        N.opt_partition_dp([1.0, 2.0], [0, 1], 2, 1.0)   # buckets do not end at nparams
    with pytest.raises(N.MatoptError):
        N.opt_plan_host_ranks([float("nan")], [1], 2, 8)


# ------------------------------------------------------------------ imbalance

def _element_even_owner(mats, bb, R):
    """The unbalanced baseline: every bucket cut into R equal element counts
    (ZeRO-1 shard boundaries) snapped to parameter boundaries."""
    sizes = [float(s.m * s.n) for s in mats]
    owner = [0] * len(mats)
    for b in range(len(bb) - 1):
        cuts = P.atomic_cuts(sizes[bb[b]:bb[b + 1]], [1.0 / R] * R)
        for r in range(R):
            for j in range(cuts[r], cuts[r + 1]):
                owner[bb[b] + j] = r
    return owner


@pytest.mark.parametrize("model", sorted(workloads.PLANNING_MODELS))
def test_alpha_balanced_partition_reduces_imbalance_on_qwen3(model):
    """Flops and memory imbalance (max / mean over ranks) of whole-matrix
    ownership: element-even ZeRO cuts versus the alpha = 1 partition. Printed
    as a table; alpha = 1 must never be worse on flops."""
    mats, bb = workloads.planning_set(model)
    K = 10 if model == "qwen3_1p7b" else 5
    costs = [P.matrix_step_cost(s.m, s.n, K, 1) for s in mats]
    mem = [4.0 * (4 * s.m * s.n + s.m * s.m + s.n * s.n) for s in mats]   # W, G, M, v + U, V (fp32)
    rows = []
    for R in (8, 16, 32, 64, 128, 256):
        base = _element_even_owner(mats, bb, R)
        bal, _ = P.alpha_balanced_partition(costs, bb, R, 1.0)
        per = lambda own, val: [sum(v for v, o in zip(val, own) if o == r) for r in range(R)]
        fb, fa = P.imbalance(per(base, costs)), P.imbalance(per(bal, costs))
        mb, ma = P.imbalance(per(base, mem)), P.imbalance(per(bal, mem))
        rows.append((R, fb, fa, mb, ma))
        assert fa <= fb + 1e-12
    print(f"\n{model}: ranks | flops imbalance even-elements -> alpha=1 | memory imbalance")
    for R, fb, fa, mb, ma in rows:
        print(f"  R={R:4d}  {fb:6.2f}x -> {fa:6.2f}x   {mb:6.2f}x -> {ma:6.2f}x")
