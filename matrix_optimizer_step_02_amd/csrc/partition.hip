// Cross-rank planners, host code only: the alpha-balanced partition of
// data-parallel buckets (Canzona page, section 3.2.1; cut points on parameter
// boundaries per section 4.2) and the capacity-capped micro-groups with
// min-heap host ranks (section 3.2.2). The contract, including the order of
// every floating-point sum, is stated with the declarations in matopt.h.
#include <algorithm>
#include <cmath>
#include <functional>
#include <numeric>
#include <queue>
#include <utility>
#include <vector>

#include "internal.h"

// Products and sums are rounded one by one, as the contract states them.
#pragma clang fp contract(off)

using namespace matopt;

namespace {

// Rank targets of one bucket given the loads so far: each rank's deficit
// below the mean of the current loads, normalised, mixed with the even split.
void bucket_shares(const std::vector<double>& load, double alpha, std::vector<double>& share) {
    const int R = (int)load.size();
    double total = 0.0;
    for (double x : load) total += x;
    const double mean = total / R;
    std::vector<double> deficit(R);
    double dsum = 0.0;
    for (int r = 0; r < R; ++r) {
        deficit[r] = std::max(0.0, mean - load[r]);
        dsum += deficit[r];
    }
    const double even = 1.0 / R;
    share.resize(R);
    for (int r = 0; r < R; ++r) {
        const double fill = dsum > 0.0 ? deficit[r] / dsum : 1.0 / R;
        share[r] = (1.0 - alpha) * even + alpha * fill;
    }
}

// Boundaries cut[0] = 0 <= cut[1] <= ... <= cut[R] = k of one bucket. The
// prefix costs are non-decreasing, so |prefix - target| is unimodal along the
// search: the scan stops at the first prefix past the target.
void atomic_cuts(const double* cost, int64_t k, const std::vector<double>& share, std::vector<int64_t>& cut) {
    const int R = (int)share.size();
    std::vector<double> prefix(k + 1);
    prefix[0] = 0.0;
    for (int64_t j = 0; j < k; ++j) prefix[j + 1] = prefix[j] + cost[j];
    const double W = prefix[k];
    cut.assign(R + 1, 0);
    double cum = 0.0;
    for (int r = 1; r < R; ++r) {
        cum += share[r - 1];
        const double target = W * cum;
        int64_t best = cut[r - 1];
        for (int64_t j = cut[r - 1]; j <= k; ++j) {
            if (std::fabs(prefix[j] - target) < std::fabs(prefix[best] - target)) best = j;
            if (prefix[j] > target) break;
        }
        cut[r] = best;
    }
    cut[R] = k;
}

}  // namespace

extern "C" opt_status opt_partition_dp(const double* cost, int64_t nparams, const int64_t* bucket_begin,
                                       int32_t nbuckets, int32_t ranks, double alpha, int32_t* owner,
                                       double* load) {
    if (!cost || !bucket_begin || !owner) return fail(OPT_EINVAL, "cost, bucket_begin and owner must not be NULL");
    if (nparams < 0 || nbuckets < 0) return fail(OPT_EINVAL, "nparams and nbuckets must be >= 0");
    if (ranks < 1) return fail(OPT_EINVAL, "ranks must be >= 1");
    if (!(alpha >= 0.0 && alpha <= 1.0)) return fail(OPT_EINVAL, "alpha must be in [0, 1]");
    if (bucket_begin[0] != 0 || bucket_begin[nbuckets] != nparams)
        return fail(OPT_EINVAL, "bucket_begin must start at 0 and end at nparams");
    for (int32_t b = 0; b < nbuckets; ++b)
        if (bucket_begin[b + 1] < bucket_begin[b]) return fail(OPT_EINVAL, "bucket_begin must be non-decreasing");
    for (int64_t i = 0; i < nparams; ++i)
        if (!(cost[i] >= 0.0) || !std::isfinite(cost[i])) return fail(OPT_EINVAL, "cost[%lld] must be finite and >= 0", (long long)i);

    std::vector<double> W(nbuckets);
    for (int32_t b = 0; b < nbuckets; ++b) {
        double s = 0.0;
        for (int64_t i = bucket_begin[b]; i < bucket_begin[b + 1]; ++i) s += cost[i];
        W[b] = s;
    }
    std::vector<int32_t> order(nbuckets);
    std::iota(order.begin(), order.end(), 0);
    std::stable_sort(order.begin(), order.end(), [&](int32_t a, int32_t b) { return W[a] > W[b]; });

    std::vector<double> L(ranks, 0.0), share;
    std::vector<int64_t> cut;
    for (int32_t b : order) {
        const int64_t lo = bucket_begin[b], k = bucket_begin[b + 1] - lo;
        bucket_shares(L, alpha, share);
        atomic_cuts(cost + lo, k, share, cut);
        for (int r = 0; r < ranks; ++r)
            for (int64_t j = cut[r]; j < cut[r + 1]; ++j) {
                owner[lo + j] = r;
                L[r] += cost[lo + j];
            }
    }
    if (load)
        for (int r = 0; r < ranks; ++r) load[r] = L[r];
    return OPT_OK;
}

extern "C" opt_status opt_plan_host_ranks(const double* cost, const uint64_t* bytes, int64_t n, int32_t ranks,
                                          uint64_t capacity_bytes, int32_t* order, int32_t* group_of,
                                          int32_t* host_of, int32_t* num_groups) {
    if (!cost || !bytes) return fail(OPT_EINVAL, "cost and bytes must not be NULL");
    if (n < 0 || n > INT32_MAX) return fail(OPT_EINVAL, "n out of range");
    if (ranks < 1) return fail(OPT_EINVAL, "ranks must be >= 1");
    for (int64_t i = 0; i < n; ++i)
        if (!(cost[i] >= 0.0) || !std::isfinite(cost[i])) return fail(OPT_EINVAL, "cost[%lld] must be finite and >= 0", (long long)i);
    const uint64_t cap = capacity_bytes ? capacity_bytes : (1ull << 29);

    std::vector<int32_t> ord(n);
    std::iota(ord.begin(), ord.end(), 0);
    std::stable_sort(ord.begin(), ord.end(), [&](int32_t a, int32_t b) { return cost[a] > cost[b]; });

    // min-heap of (load in the current group, rank)
    typedef std::pair<double, int32_t> Slot;
    std::priority_queue<Slot, std::vector<Slot>, std::greater<Slot>> heap;
    int32_t g = -1;
    uint64_t used = 0;
    int64_t members = 0;
    for (int64_t k = 0; k < n; ++k) {
        const int32_t i = ord[k];
        if (g < 0 || (members > 0 && (used > cap || bytes[i] > cap - used))) {
            ++g;
            used = 0;
            members = 0;
            heap = decltype(heap)();
            for (int32_t r = 0; r < ranks; ++r) heap.push(Slot(0.0, r));
        }
        Slot s = heap.top();
        heap.pop();
        s.first += cost[i];
        heap.push(s);
        used += bytes[i];
        ++members;
        if (order) order[k] = i;
        if (group_of) group_of[i] = g;
        if (host_of) host_of[i] = s.second;
    }
    if (num_groups) *num_groups = g + 1;
    return OPT_OK;
}
