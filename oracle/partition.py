"""Plain CPU oracle of the cross-rank planners (host logic, float64).

TEST INFRASTRUCTURE. Only ``tests/`` may import or call this module; the
library's own planners (``opt_partition_dp``, ``opt_plan_host_ranks``) share
no code with it.

Source: the Canzona page (aitangshan.cn), cited by section:

* section 2.1: atomicity -- a matrix optimizer needs whole matrices, so a
  parameter is never split between ranks.
* section 3.2.1: alpha-balanced greedy LPT partition for data parallelism.
  Buckets are taken in decreasing order of processing time. For each bucket
  the gap between every rank's load and the ideal mean is computed; the
  bucket's per-rank target shares mix an even split (alpha -> 0) with shares
  that fill the gaps (alpha -> 1); the cut points are then placed on
  parameter boundaries, and the loads are updated.
* section 3.2.2: micro-group scheduling for tensor parallelism. All parameters
  are sorted by cost, largest first; each is tentatively added to the current
  micro-group, whose loads over the host ranks are simulated with a min-heap;
  if the group's capacity would be exceeded the addition is rolled back and a
  new group is opened.
* section 4.2: geometric alignment -- the physical order of parameters is
  kept; only the logical cut points move.
* section 6.1: alpha = 1 is usually best; 512 MB - 1 GB micro-groups.

Readings where the section is silent or garbled (each listed in the design doc):

* the "ideal mean" against which a rank's deficit is measured is the mean
  of the loads before the bucket, sum(L) / R, as the section's listing
  computes it (the comparison in the listing's test of the deficit sum is
  lost in the extraction; "greater than zero" is the only reading that
  avoids a division by zero);
  with alpha = 1 a bucket therefore goes to the ranks below that mean in
  proportion to their deficits, and to every rank evenly when none trails
  (the first bucket, or equal loads);
* a bucket's parameters keep their physical order and rank r receives one
  consecutive range, ranks in increasing order (ZeRO-1 geometry); the cut
  for boundary r is the parameter boundary whose prefix cost is nearest to
  W_b times the cumulative target share of ranks < r, not before the
  previous cut; ties go to the earlier boundary;
* buckets of equal cost keep their input order (stable sort);
* the capacity of a micro-group bounds the sum of its parameters' bytes; a
  parameter larger than the capacity forms a group of its own; the min-heap
  assigns each parameter of a group to the host rank with the least load in
  that group so far, ties to the lowest rank index.

Every floating-point sum runs left to right in the order written here, so that
an implementation that keeps the same order reproduces the integer results
exactly.
"""

from __future__ import annotations

from typing import List, Sequence, Tuple

__all__ = ["bucket_shares", "atomic_cuts", "alpha_balanced_partition", "micro_groups_host_ranks",
           "imbalance", "matrix_step_cost"]


def matrix_step_cost(m: int, n: int, K: int, power_iters: int) -> float:
    """Flops of one step of the rotated-basis method on an m x n matrix: the
    two-sided rotations of G and M and the rotation back, 6 m n (m + n), plus
    the basis refresh amortised over K steps, p [8 m n r + (8/3)(m^3 + n^3)]."""
    r = min(m, n)
    c = 6.0 * m * n * (m + n)
    if K > 0:
        c += power_iters * (8.0 * m * n * r + (8.0 / 3.0) * (float(m) ** 3 + float(n) ** 3)) / K
    return c


def bucket_shares(loads: Sequence[float], W: float, alpha: float) -> List[float]:
    """Target share of each rank for a bucket of cost W (section 3.2.1):
    deficits against the mean of the current loads, sum(L) / R, normalised
    to fill shares; mixed with the even split by alpha. W does not enter the
    shares (it scales the cut targets in atomic_cuts)."""
    R = len(loads)
    total = 0.0
    for x in loads:
        total += x
    mean = total / R
    deficits = [max(0.0, mean - x) for x in loads]
    dsum = 0.0
    for d in deficits:
        dsum += d
    fill = [d / dsum for d in deficits] if dsum > 0.0 else [1.0 / R] * R
    even = 1.0 / R
    return [(1.0 - alpha) * even + alpha * f for f in fill]


def atomic_cuts(costs: Sequence[float], shares: Sequence[float]) -> List[int]:
    """Cut positions j_0 = 0 <= j_1 <= ... <= j_R = k on parameter boundaries
    (section 3.2.1, 4.2): rank r receives parameters [j_r, j_{r+1})."""
    k = len(costs)
    R = len(shares)
    prefix = [0.0]
    for c in costs:
        prefix.append(prefix[-1] + c)
    W = prefix[k]
    cuts = [0]
    cum = 0.0
    for r in range(1, R):
        cum += shares[r - 1]
        target = W * cum
        best = cuts[-1]
        for j in range(cuts[-1], k + 1):
            if abs(prefix[j] - target) < abs(prefix[best] - target):
                best = j
        cuts.append(best)
    cuts.append(k)
    return cuts


def alpha_balanced_partition(costs: Sequence[float], bucket_begin: Sequence[int], R: int,
                             alpha: float) -> Tuple[List[int], List[float]]:
    """owner[i] of every parameter and the final per-rank loads.

    ``bucket_begin`` has one entry per bucket plus the end (bucket b holds
    parameters bucket_begin[b] .. bucket_begin[b+1]-1)."""
    nb = len(bucket_begin) - 1
    W = []
    for b in range(nb):
        s = 0.0
        for i in range(bucket_begin[b], bucket_begin[b + 1]):
            s += costs[i]
        W.append(s)
    order = sorted(range(nb), key=lambda b: -W[b])   # stable: equal costs keep input order
    loads = [0.0] * R
    owner = [-1] * len(costs)
    for b in order:
        lo, hi = bucket_begin[b], bucket_begin[b + 1]
        shares = bucket_shares(loads, W[b], alpha)
        cuts = atomic_cuts(costs[lo:hi], shares)
        for r in range(R):
            for j in range(cuts[r], cuts[r + 1]):
                owner[lo + j] = r
                loads[r] += costs[lo + j]
    return owner, loads


def micro_groups_host_ranks(costs: Sequence[float], nbytes: Sequence[int], R: int,
                            capacity: int) -> Tuple[List[int], List[int], List[int], int]:
    """(order, group_of, host_of, num_groups) of section 3.2.2."""
    n = len(costs)
    order = sorted(range(n), key=lambda i: -costs[i])
    group_of = [-1] * n
    host_of = [-1] * n
    g = -1
    used = 0
    loads: List[float] = []
    members = 0
    for i in order:
        if g < 0 or (members > 0 and used + nbytes[i] > capacity):
            g += 1
            used = 0
            loads = [0.0] * R
            members = 0
        h = min(range(R), key=lambda r: (loads[r], r))
        loads[h] += costs[i]
        used += nbytes[i]
        members += 1
        group_of[i] = g
        host_of[i] = h
    return order, group_of, host_of, g + 1


def imbalance(values: Sequence[float]) -> float:
    """max / mean (1.0 = perfectly balanced)."""
    mean = sum(values) / len(values)
    return max(values) / mean if mean > 0 else 1.0
