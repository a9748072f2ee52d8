// Host-side checks of the C ABI under AddressSanitizer and UBSan.
//
// Test infrastructure: built by tests/test_asan_host.py with the library's
// sources compiled with -fsanitize=address,undefined on their host side (no
// kernel is launched, no GPU is touched). Everything called here returns before any
// HIP call: the planners, the workspace sizing of every flag combination,
// and the argument checks of create and the building blocks. A sanitizer
// report aborts the run with a non-zero status.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <random>
#include <algorithm>
#include <vector>

#include "matopt.h"

namespace {

int failures = 0;

void expect(bool ok, const char* what) {
    if (!ok) {
        std::fprintf(stderr, "FAILED: %s (%s)\n", what, opt_last_error());
        ++failures;
    }
}

opt_hparams hp(uint32_t flags = 0, int32_t ns = 0) {
    opt_hparams h{};
    h.beta1 = 0.9f;
    h.beta2 = 0.999f;
    h.eps = 1e-8f;
    h.lr = 1e-3f;
    h.K = 10;
    h.power_iters = 1;
    h.flags = flags;
    h.ns_iters = ns;
    return h;
}

opt_matrix_desc desc(int64_t m, int64_t n, int32_t dtype, uintptr_t base) {
    opt_matrix_desc d{};
    d.m = m;
    d.n = n;
    d.M_dtype = dtype;
    if (base) {
        const uintptr_t step = uintptr_t(1) << 32;
        d.W = (float*)(base);
        d.G = (const float*)(base + step);
        d.M = (void*)(base + 2 * step);
        d.v = (float*)(base + 3 * step);
        d.U = (float*)(base + 4 * step);
        d.V = (float*)(base + 5 * step);
    }
    return d;
}

// The Qwen3-1.7B-shaped set: 28 layers of q, k, v, o, up, gate, down.
std::vector<opt_matrix_desc> qwen3_1p7b(int32_t dtype) {
    const int64_t s[7][2] = {{2048, 2048}, {2048, 1024}, {2048, 1024}, {2048, 2048},
                             {2048, 6144}, {2048, 6144}, {6144, 2048}};
    std::vector<opt_matrix_desc> out;
    for (int l = 0; l < 28; ++l)
        for (auto& x : s) out.push_back(desc(x[0], x[1], dtype, 0));
    return out;
}

void planners() {
    std::mt19937_64 rng(7);
    std::uniform_real_distribution<double> u(0.0, 10.0);
    for (int c = 0; c < 300; ++c) {
        const int R = 1 + (int)(rng() % 12), nb = (int)(rng() % 10);
        std::vector<int64_t> bb{0};
        std::vector<double> cost;
        for (int b = 0; b < nb; ++b) {
            const int k = (int)(rng() % 13);
            for (int i = 0; i < k; ++i) cost.push_back((rng() % 4 == 0) ? 0.0 : u(rng));
            bb.push_back((int64_t)cost.size());
        }
        const int64_t np = (int64_t)cost.size();
        cost.push_back(0.0);   // the arrays must not be NULL even when empty
        std::vector<int32_t> owner(np + 1);
        std::vector<double> load(R);
        expect(opt_partition_dp(cost.data(), np, bb.data(), nb, R, 0.1 * (c % 11), owner.data(),
                                load.data()) == OPT_OK, "partition");
        const int64_t n = (int64_t)(rng() % 40);
        std::vector<double> c2(n + 1);
        std::vector<uint64_t> bytes(n + 1);
        for (int64_t i = 0; i < n; ++i) {
            c2[i] = u(rng);
            bytes[i] = rng() % 64;
        }
        std::vector<int32_t> order(n + 1), gof(n + 1), host(n + 1);
        int32_t ng = 0;
        expect(opt_plan_host_ranks(c2.data(), bytes.data(), n, R, 1 + rng() % 100, order.data(), gof.data(),
                                   host.data(), &ng) == OPT_OK, "host ranks");
    }
    double one = 1.0;
    int64_t bad_bb[2] = {0, 2};
    int32_t owner[2];
    expect(opt_partition_dp(&one, 1, bad_bb, 1, 2, 1.0, owner, nullptr) == OPT_EINVAL, "partition: bad buckets");
    expect(opt_partition_dp(&one, 1, bad_bb, 1, 0, 1.0, owner, nullptr) == OPT_EINVAL, "partition: no ranks");
}

void plans_and_sizes() {
    for (int32_t dt : {OPT_F32, OPT_BF16}) {
        std::vector<opt_matrix_desc> d = qwen3_1p7b(dt);
        std::vector<int32_t> order(d.size()), gof(d.size());
        int32_t ng = 0;
        opt_hparams h = hp();
        expect(opt_plan(d.data(), (int32_t)d.size(), &h, order.data(), gof.data(), &ng) == OPT_OK && ng == 11,
               "plan: 11 groups");
        const uint32_t flag_sets[] = {0u,
                                      OPT_FLAG_FP32_MFMA,
                                      OPT_FLAG_ROTATED_MOMENTUM,
                                      OPT_FLAG_BF16_ROTATION,
                                      OPT_FLAG_BF16_ROTATION | OPT_FLAG_ROTATED_MOMENTUM,
                                      OPT_FLAG_MUON,
                                      OPT_FLAG_MUON | OPT_FLAG_FP32_MFMA};
        for (uint32_t f : flag_sets) {
            opt_hparams hf = hp(f, (f & OPT_FLAG_MUON) ? 3 : 0);
            uint64_t bytes = 0;
            expect(opt_group_workspace_size(d.data(), (int32_t)d.size(), &hf, &bytes) == OPT_OK && bytes > 0,
                   "workspace size");
            uint64_t parts[4] = {};
            expect(opt_group_workspace_parts(d.data(), (int32_t)d.size(), &hf, parts) == OPT_OK &&
                       parts[0] + std::max(parts[1] + parts[2], parts[3]) == bytes,
                   "workspace parts");
        }
    }
    // ragged shapes, every flag set
    std::vector<opt_matrix_desc> r = {desc(37, 53, OPT_F32, 0), desc(130, 67, OPT_BF16, 0), desc(1, 9, OPT_F32, 0),
                                      desc(16384, 64, OPT_BF16, 0)};
    for (uint32_t f : {0u, 1u, 2u, 3u, 8u}) {
        opt_hparams hf = hp(f);
        uint64_t bytes = 0;
        expect(opt_group_workspace_size(r.data(), (int32_t)r.size(), &hf, &bytes) == OPT_OK, "ragged size");
    }
    uint64_t b = 0;
    expect(opt_orthonormalize_workspace_size(4096, &b) == OPT_OK && b > 0, "qr workspace");
    expect(opt_orthonormalize_workspace_size(0, &b) == OPT_EINVAL, "qr workspace d = 0");
}

void argument_errors() {
    opt_hparams h = hp();
    opt_group_t g = nullptr;
    const uintptr_t base = uintptr_t(1) << 40, ws = uintptr_t(1) << 44;
    std::vector<opt_matrix_desc> d = {desc(8, 8, OPT_F32, base), desc(8, 8, OPT_F32, base + (uintptr_t(6) << 32))};
    uint64_t need = 0;
    expect(opt_group_workspace_size(d.data(), 2, &h, &need) == OPT_OK, "size");
    expect(opt_group_create(d.data(), 2, &h, (void*)ws, need - 1, nullptr, &g) == OPT_ENOWS, "ENOWS");
    expect(opt_group_create(d.data(), 2, &h, (void*)(ws + 8), need, nullptr, &g) == OPT_EINVAL, "unaligned ws");
    opt_matrix_desc o = d[1];
    o.W = d[0].W + 3;
    std::vector<opt_matrix_desc> ov = {d[0], o};
    expect(opt_group_create(ov.data(), 2, &h, (void*)ws, need, nullptr, &g) == OPT_EINVAL, "overlap");
    std::vector<opt_matrix_desc> tail = {d[0]};
    tail[0].W = (float*)(ws - 64);
    expect(opt_group_create(tail.data(), 1, &h, (void*)ws, need, nullptr, &g) == OPT_EINVAL, "tail in workspace");
    opt_hparams bad = hp();
    bad.beta1 = 1.f;
    expect(opt_group_create(d.data(), 2, &bad, (void*)ws, need, nullptr, &g) == OPT_EINVAL, "beta1");
    bad = hp(1u << 9);
    expect(opt_group_create(d.data(), 2, &bad, (void*)ws, need, nullptr, &g) == OPT_EINVAL, "flags");
    expect(g == nullptr, "no group on error");
    expect(opt_group_step(nullptr, nullptr) == OPT_EINVAL, "null step");
    opt_group_destroy(nullptr);
    expect(opt_gemm(0, 0, -1, 4, 4, 1.f, (void*)base, 0, 4, (void*)base, 0, 4, 0.f, (float*)base, 4, nullptr) ==
               OPT_EINVAL, "gemm negative");
    expect(opt_gemm_bf16(4, 4, 7, 1.f, (void*)base, 8, (void*)base, 8, 0.f, (void*)base, 0, 4, nullptr) == OPT_EINVAL,
           "gemm16 K");
    expect(opt_orthonormalize_static(nullptr, nullptr, OPT_STATIC_MAX_DIM + 1, nullptr) == OPT_EUNSUPPORTED,
           "static qr: order");
    expect(std::strlen(opt_last_error()) > 0, "error text");
}

}  // namespace

int main() {
    planners();
    plans_and_sizes();
    argument_errors();
    std::printf("host checks: %d failures\n", failures);
    return failures ? 1 : 0;
}
