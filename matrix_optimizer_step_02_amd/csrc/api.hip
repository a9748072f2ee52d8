// C ABI of the rotated-basis matrix-optimizer step: argument checks, the
// micro-group planner, the workspace layout and the per-step launch schedule.
//
// Planner (Canzona page, section 3.2.2 micro-group scheduling; section 6.1
// group size): matrices are ordered by cost m*n*(m+n) descending, ties by
// input position (a stable longest-processing-time order), and packed next-fit
// into micro-groups whose fp32 gradient payload sum(4 m n) stays within the
// capacity; a new group opens when the next matrix does not fit. Inside one
// group every phase is a single grouped launch whose problems are again in
// LPT order (costliest k first), so the hardware dispatcher hands the long
// tiles out first.
//
// Workspace: [device work lists of every group | scratch of one group]. The
// scratch of a group is either its rotation buffers (U^T G, U^T M, G~, m~;
// 4 m n floats per matrix, reused for U u and u) or its refresh buffers (Gram
// products, the QR inputs Z and the QR scratch), never both at once, and the
// groups run one after another on the stream, so one maximum-sized scratch
// serves them all.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <numeric>
#include <string>
#include <utility>
#include <vector>

#include "matopt.h"
#include "variant_bf16.h"
#include "variant_muon.h"

using namespace matopt;

namespace {
thread_local std::string g_err;
}  // namespace

opt_status matopt::fail(opt_status st, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return st;
}

namespace {

opt_status hip_fail(hipError_t e, const char* where) {
    return fail(OPT_EHIP, "%s: %s", where, hipGetErrorString(e));
}

constexpr uint64_t kAlign = 256;
constexpr uint64_t align_up(uint64_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

struct Mat {
    opt_matrix_desc d;
    int idx;
    double cost;
    bool bf16;
    // bf16-rotation variant: bf16 copies of U, U^T (m x m8) and V, V^T (n x n8)
    uint16_t *Ub = nullptr, *Utb = nullptr, *Vb = nullptr, *Vtb = nullptr;
    // fp32 rotations: U^T (m x m), so that U^T [G | M] reads k-contiguous rows
    float* Ut = nullptr;
    // fp32 rotations of a bf16 M (m, n multiples of 8): the product of M's
    // rotation chain with the larger flop count runs as three bf16 products
    // against exact bf16 pieces of the basis. Tall (m > n): U^T M with the
    // pieces of U^T; otherwise M V with the pieces of V^T. Bp holds the three
    // pieces of that transposed basis (d x d each, d = m or n).
    uint16_t* Bp = nullptr;
    bool tall = false;
};

// Byte offsets into the table image (host) / table region (device).
struct GemmLaunch {
    int variant = 0;
    int cfg = 0;     // index into kGemmCfgs
    int nprob = 0;
    int total_tiles = 0;
    uint64_t probs = 0;
    uint64_t tb = 0;
};
struct EwLaunch {
    int nseg = 0;
    int64_t chunks = 0;
    uint64_t segs = 0;
};
struct Gemm16Launch {
    bool out16 = false;
    int cfg = 0;     // index into kGemm16Cfgs
    int nprob = 0;
    int total_tiles = 0;
    uint64_t probs = 0;
    uint64_t tb = 0;
};
struct PackLaunch {
    int njobs = 0;
    int64_t chunks = 0;
    uint64_t jobs = 0;
};
struct QrBatch {
    int njobs = 0;
    uint64_t jobs = 0;
    std::vector<int> np;   // panels per job, descending
    std::vector<int> d;    // order per job, descending
    int max_d = 0;
    // grouped GEMM launches of the outer blocks: [block][step] -> launches
    std::vector<std::vector<std::vector<GemmLaunch>>> fact, qform;
};
struct CopyLaunch {
    int n = 0;
    uint64_t jobs = 0;
    int max_d = 0;
};

struct Group {
    std::vector<int> mats;   // indices into opt_group_s::mats, LPT order
    EwLaunch mom, adam;
    std::vector<GemmLaunch> rot_left, rot_right, back_left, back_right;
    // M's pieced bf16 products (matrices with Bp), and the M^T copies that
    // the tall ones read
    std::vector<Gemm16Launch> rot_m16;
    uint64_t mt_split = 0;
    int mt_nsplit = 0, mt_tiles = 0;
    // with the carried rotated momentum: the step that recomputes m~ = U^T M V
    // into Mt (rot_left as above), and the step that carries it (G only)
    std::vector<GemmLaunch> rot_right_re, rot_left_c, rot_right_c;
    EwLaunch adam_re, adam_c;
    // bf16 rotations: S = (X V)^T for X in {G, M}, then U^T S^T into G~, m~;
    // P = (u V^T)^T, then W -= lr U P^T. Matrices with n % 8 == 0 take the
    // fused elementwise launches (bf16 side outputs), others the plain ones
    // followed by packs to a padded row stride.
    std::vector<Gemm16Launch> r16_right, r16_left, r16_back_right, r16_back_left;
    EwLaunch mom16, adam16;
    EwLaunch mom_r, adam_r;   // ragged matrices
    // with the carried rotated momentum as well: the step that carries m~
    // (G alone rotated, m~ advanced in the Adam kernel) and the step that
    // recomputes it into Mt
    std::vector<Gemm16Launch> r16_right_c, r16_left_c, r16_left_re;
    EwLaunch adam16_c, adam16_re, adam_r_c, adam_r_re;
    PackLaunch pack_in, pack_u;
    // orthogonalised momentum (OPT_FLAG_MUON): MuonSeg list (EwLaunch of
    // MuonSeg), the Gram and product launches of one Newton-Schulz step, and
    // the norm partials and inverse norms in the scratch
    EwLaunch mu;
    std::vector<GemmLaunch> mu_gram, mu_prod;
    double* mu_part = nullptr;
    float* mu_inv = nullptr;
    uint64_t rot_bytes = 0;
};

// One Newton-Schulz row chunk of a refresh batch's bases: P = X[rows] G
// (K-chunk steps), then X[rows] = 1.5 X[rows] - 0.5 P.
struct NsChunk {
    std::vector<std::vector<GemmLaunch>> prod;
    uint64_t jobs = 0;
    int njobs = 0;
    int64_t max_n = 0;
};

// Matrices refreshed together: Gram products, completion copies, QR jobs.
// The same batch (and scratch layout) serves the state checks and the
// re-orthonormalisation: gram forms X^T X of every basis in its QR input
// buffer Z.
struct RefreshBatch {
    std::vector<int> mats;
    std::vector<std::vector<GemmLaunch>> prod1, prod2;   // K-chunk steps, run in order
    CopyLaunch comp;
    QrBatch qr;
    uint64_t ref_bytes = 0;
    std::vector<std::vector<GemmLaunch>> gram;
    uint64_t drift_jobs = 0;
    int ndrift = 0, drift_max_d = 0;
    std::vector<NsChunk> ns;
    // bases stored in 16 bits: widen U, V into the refresh's fp32 copies
    // before the first pass, round them back after the last
    int nwiden = 0;
    int64_t widen_chunks = 0, round_chunks = 0;
    uint64_t widen = 0, round16 = 0;
};

// Append-only image of device tables with 256-byte aligned entries.
struct Image {
    std::vector<uint8_t> bytes;
    template <class T>
    uint64_t put(const std::vector<T>& v) {
        const uint64_t off = align_up(bytes.size());
        bytes.resize(off + sizeof(T) * v.size());
        if (!v.empty()) memcpy(bytes.data() + off, v.data(), sizeof(T) * v.size());
        return off;
    }
};

}  // namespace

struct opt_group_s {
    std::vector<Mat> mats;
    opt_hparams hp{};
    int64_t t = 0;
    std::vector<Group> groups;
    std::vector<RefreshBatch> rbatches;
    char* ws = nullptr;
    uint64_t ws_bytes = 0;
    Image img;
    uint64_t table_bytes = 0, scratch_bytes = 0;
    // the largest refresh batch's buffers, which start where the copies of
    // the bases start and overlay them and the scratch
    uint64_t refresh_bytes_max = 0;
    // copies of the bases after the tables, before the scratch: bf16 U, U^T,
    // V, V^T (bf16-rotation variant) or fp32 U^T (fp32 rotations), their
    // conversion launch, and whether they match U, V
    uint64_t bases_bytes = 0;
    uint64_t basis_jobs = 0;
    int basis_njobs = 0, basis_tiles = 0;
    uint64_t transpose_jobs = 0;
    int transpose_njobs = 0, transpose_tiles = 0;
    uint64_t pieces_jobs = 0;   // bf16 pieces of U^T or V^T (Mat::Bp)
    int pieces_njobs = 0, pieces_tiles = 0;
    bool copies_valid = false;
    // state checks: one scan over every matrix (partials at the start of the
    // scratch), per-matrix records in the table region
    uint64_t health_segs = 0, health_out = 0;
    int health_nseg = 0;
    int64_t health_chunks = 0;
    int device = 0;
    bool mt_valid = false;   // the carried rotated momentum matches U, V (OPT_FLAG_ROTATED_MOMENTUM)
    // timing: events are created when timing is enabled (never inside a
    // step); a scope that finds the pool used up is not recorded and is
    // reported by read_timing, which folds the records into the totals and
    // frees the pool again
    bool timing = false;
    bool timing_overflow = false;
    std::vector<hipEvent_t> pool;
    size_t pool_used = 0;
    double acc_ms[OPT_NUM_PHASES] = {};
    int64_t acc_kernels[OPT_NUM_PHASES] = {};
    std::vector<double> acc_group_ms;   // per micro-group, every phase of its scopes
    struct Rec {
        int phase;
        int group;   // micro-group of the scope, -1 for the refresh batches and the basis copies
        hipEvent_t b, e;
        int kernels;
    };
    std::vector<Rec> recs;
    int kernels_in_scope = 0;   // kernels launched since the current phase scope opened
};

namespace {

// ---------------------------------------------------------------- checks ----

opt_status check_hparams(const opt_hparams* hp) {
    if (!hp) return fail(OPT_EINVAL, "hparams is NULL");
    if (!(hp->beta1 >= 0.f && hp->beta1 < 1.f)) return fail(OPT_EINVAL, "beta1 must be in [0, 1)");
    if (!(hp->beta2 >= 0.f && hp->beta2 < 1.f)) return fail(OPT_EINVAL, "beta2 must be in [0, 1)");
    if (!(hp->eps > 0.f) || !std::isfinite(hp->eps)) return fail(OPT_EINVAL, "eps must be finite and > 0");
    if (!std::isfinite(hp->lr)) return fail(OPT_EINVAL, "lr must be finite");
    if (hp->K < 0) return fail(OPT_EINVAL, "K must be >= 0");
    if (hp->power_iters < 1) return fail(OPT_EINVAL, "power_iters must be >= 1");
    if (hp->flags & ~(uint32_t)(OPT_FLAG_ROTATED_MOMENTUM | OPT_FLAG_BF16_ROTATION | OPT_FLAG_MUON |
                                OPT_FLAG_FP32_MFMA | OPT_FLAG_BF16_BASES))
        return fail(OPT_EINVAL, "unknown bits in flags");
    if ((hp->flags & OPT_FLAG_BF16_BASES) && !(hp->flags & OPT_FLAG_BF16_ROTATION))
        return fail(OPT_EINVAL, "OPT_FLAG_BF16_BASES needs OPT_FLAG_BF16_ROTATION");
    if ((hp->flags & OPT_FLAG_MUON) && (hp->flags & ~(uint32_t)OPT_FLAG_FP32_MFMA) != OPT_FLAG_MUON)
        return fail(OPT_EUNSUPPORTED, "OPT_FLAG_MUON combines with OPT_FLAG_FP32_MFMA only");
    if ((hp->flags & OPT_FLAG_MUON) && hp->ns_iters < 1)
        return fail(OPT_EINVAL, "ns_iters must be >= 1 with OPT_FLAG_MUON");
    return OPT_OK;
}

uint64_t capacity_of(const opt_hparams* hp) {
    return hp->capacity_bytes ? hp->capacity_bytes : (1ull << 29);
}

// The refresh cap: the caller's, else the largest of 4 GiB, `overlay` (the
// bytes of the copies of the bases and the step's scratch, which a refresh
// batch's buffers overlay: the copies are rebuilt after every refresh) and
// `state` (the bytes of the caller's tensors), so that by default the
// workspace is no larger than the larger of the state it serves and the
// copies and scratch of a step, unless one matrix's refresh alone is.
uint64_t refresh_capacity_of(const opt_hparams* hp, uint64_t overlay, uint64_t state) {
    if (hp->refresh_capacity_bytes) return hp->refresh_capacity_bytes;
    return std::max<uint64_t>(std::max<uint64_t>(4ull << 30, overlay), state);
}

// Bytes of the caller-owned tensors of a group: W, G, v (fp32), M, U, V, and
// Mt with the carried rotated momentum.
uint64_t state_bytes(const opt_group_s* g) {
    uint64_t b = 0;
    const bool b16 = g->hp.flags & OPT_FLAG_BF16_BASES, muon = g->hp.flags & OPT_FLAG_MUON;
    const bool rmf = g->hp.flags & OPT_FLAG_ROTATED_MOMENTUM;
    for (const Mat& M : g->mats) {
        const uint64_t m = (uint64_t)M.d.m, n = (uint64_t)M.d.n, mn = m * n;
        b += mn * (8 + (muon ? 0 : 4) + (M.bf16 ? 2 : 4) + (rmf ? 4 : 0));
        if (!muon) b += (b16 ? 2 : 4) * (m * m + n * n);
    }
    return b;
}

struct Span {
    uintptr_t lo, hi;
    int mat;
    const char* what;
};

// `spans_out`, when given, receives the byte range of every tensor (with
// need_ptrs), sorted by start address.
opt_status check_descs(const opt_matrix_desc* d, int32_t count, const opt_hparams* hp,
                       bool need_ptrs, std::vector<Span>* spans_out = nullptr) {
    if (!d) return fail(OPT_EINVAL, "descs is NULL");
    if (count < 1 || count > OPT_MAX_MATRICES)
        return fail(OPT_EINVAL, "count must be in [1, %d]", OPT_MAX_MATRICES);
    opt_status st = check_hparams(hp);
    if (st) return st;
    const uint64_t cap = capacity_of(hp);
    std::vector<Span> spans;
    for (int i = 0; i < count; ++i) {
        const opt_matrix_desc& x = d[i];
        if (x.m < 1 || x.n < 1) return fail(OPT_EINVAL, "matrix %d: m and n must be >= 1", i);
        if (x.m > OPT_MAX_DIM || x.n > OPT_MAX_DIM)
            return fail(OPT_EUNSUPPORTED, "matrix %d: m and n must be <= %d", i, OPT_MAX_DIM);
        if (x.M_dtype != OPT_F32 && x.M_dtype != OPT_BF16)
            return fail(OPT_EUNSUPPORTED, "matrix %d: M_dtype must be OPT_F32 or OPT_BF16", i);
        if ((uint64_t)4 * x.m * x.n > cap)
            return fail(OPT_EINVAL,
                        "matrix %d: its gradient payload 4*m*n = %llu exceeds the micro-group "
                        "capacity %llu (a matrix is never split)",
                        i, (unsigned long long)(4ull * x.m * x.n), (unsigned long long)cap);
        if (!need_ptrs) continue;
        const bool muon = hp->flags & OPT_FLAG_MUON;
        if (!x.W || !x.G || !x.M || (!muon && (!x.v || !x.U || !x.V)))
            return fail(OPT_EINVAL, "matrix %d: a tensor pointer is NULL", i);
        const bool rm = hp->flags & OPT_FLAG_ROTATED_MOMENTUM;
        if (rm != (x.Mt != nullptr))
            return fail(OPT_EINVAL, "matrix %d: Mt must be set exactly when OPT_FLAG_ROTATED_MOMENTUM is", i);
        const uint64_t mn = (uint64_t)x.m * x.n;
        const uint64_t esz = x.M_dtype == OPT_BF16 ? 2 : 4;
        const uint64_t bsz = (hp->flags & OPT_FLAG_BF16_BASES) ? 2 : 4;   // U, V
        auto add = [&](const void* p, uint64_t bytes, const char* what) {
            spans.push_back({(uintptr_t)p, (uintptr_t)p + bytes, i, what});
        };
        add(x.W, 4 * mn, "W");
        add(x.G, 4 * mn, "G");
        add(x.M, esz * mn, "M");
        if (x.v) add(x.v, 4 * mn, "v");
        if (x.U) add(x.U, bsz * x.m * x.m, "U");
        if (x.V) add(x.V, bsz * x.n * x.n, "V");
        if (x.Mt) add(x.Mt, 4 * mn, "Mt");
        if (!aligned(x.W, 4) || !aligned(x.G, 4) || !aligned(x.v, 4) || !aligned(x.U, bsz) ||
            !aligned(x.V, bsz) || !aligned(x.M, esz) || !aligned(x.Mt, 4))
            return fail(OPT_EINVAL, "matrix %d: a tensor pointer is not aligned to its element", i);
        if ((hp->flags & OPT_FLAG_BF16_BASES) && (!aligned(x.U, 16) || !aligned(x.V, 16)))
            return fail(OPT_EINVAL, "matrix %d: with OPT_FLAG_BF16_BASES, U and V must be 16-byte aligned", i);
    }
    if (need_ptrs) {
        std::sort(spans.begin(), spans.end(), [](const Span& a, const Span& b) { return a.lo < b.lo; });
        for (size_t k = 1; k < spans.size(); ++k)
            if (spans[k].lo < spans[k - 1].hi)
                return fail(OPT_EINVAL, "tensors overlap: %s of matrix %d and %s of matrix %d",
                            spans[k - 1].what, spans[k - 1].mat, spans[k].what, spans[k].mat);
    }
    if (spans_out) *spans_out = std::move(spans);
    return OPT_OK;
}

// --------------------------------------------------------------- planning ----

void plan_groups(const opt_matrix_desc* d, int32_t count, const opt_hparams* hp,
                 std::vector<int>& order, std::vector<std::vector<int>>& groups) {
    order.resize(count);
    std::iota(order.begin(), order.end(), 0);
    auto cost = [&](int i) { return (double)d[i].m * (double)d[i].n * (double)(d[i].m + d[i].n); };
    std::stable_sort(order.begin(), order.end(), [&](int a, int b) { return cost(a) > cost(b); });
    const uint64_t cap = capacity_of(hp);
    groups.clear();
    uint64_t used = 0;
    for (int i : order) {
        const uint64_t bytes = 4ull * d[i].m * d[i].n;
        if (groups.empty() || used + bytes > cap) {
            groups.emplace_back();
            used = 0;
        }
        groups.back().push_back(i);
        used += bytes;
    }
}

// Vector loads need 4-element groups that never straddle the end of a row.
uint32_t vec_flags(const void* A, int64_t lda, int64_t a_cols, bool a_bf16, const void* B, int64_t ldb,
                   int64_t b_cols, bool b_bf16) {
    uint32_t f = 0;
    if (lda % 4 == 0 && a_cols % 4 == 0 && aligned(A, a_bf16 ? 8 : 16)) f |= GF_A_VEC;
    if (ldb % 4 == 0 && b_cols % 4 == 0 && aligned(B, b_bf16 ? 8 : 16)) f |= GF_B_VEC;
    return f;
}

struct PGemm {
    GemmProb p;
    int variant;
};

void set_tiles(GemmProb& p, int cfg) {
    p.tiles_m = (p.M + kGemmCfgs[cfg].bm - 1) / kGemmCfgs[cfg].bm;
    p.tiles_n = (p.N + kGemmCfgs[cfg].bn - 1) / kGemmCfgs[cfg].bn;
}

int tiles_of(const std::vector<GemmProb>& probs, int cfg) {
    int t = 0;
    for (GemmProb q : probs) {
        set_tiles(q, cfg);
        t += q.tiles_m * q.tiles_n;
    }
    return t;
}

// Large tiles when the launch has enough of them to fill the GPU, except for
// launches whose products are all short in K (the QR's C -= Yb W2 with
// K = 256): there a tile's epilogue (C read and written) is long against its
// few slabs, and the small tile's three workgroups per CU overlap one's
// epilogue with the others' MFMAs (a refresh of the Qwen3-1.7B set 779 ->
// 755 ms; 0 turns this off).
#ifndef MATOPT_SMALL_TILE_MAX_K
#define MATOPT_SMALL_TILE_MAX_K 256
#endif
int choose_cfg(const std::vector<GemmProb>& probs) {
    if (MATOPT_SMALL_TILE_MAX_K > 0) {
        bool short_k = !probs.empty();
        for (const GemmProb& q : probs) short_k = short_k && q.K <= MATOPT_SMALL_TILE_MAX_K;
        if (short_k) return 0;
    }
    return tiles_of(probs, 1) >= kGemmLargeMinTiles ? 1 : 0;
}

// Period of a pieced product's k range: K rounded up to whole 64-deep slabs.
int32_t kper16(int64_t K) { return (int32_t)std::max<int64_t>(64, (K + 63) / 64 * 64); }

// bf16 NT products (C = alpha A B^T + beta C, k contiguous in both operands).
Gemm16Prob g16(const void* A, int64_t lda, const void* B, int64_t ldb, void* C, int64_t ldc, int64_t M,
               int64_t N, int64_t K, float alpha, float beta, int64_t pad_n) {
    Gemm16Prob p{};
    p.A = (const uint16_t*)A;
    p.B = (const uint16_t*)B;
    p.C = C;
    p.lda = lda;
    p.ldb = ldb;
    p.ldc = ldc;
    p.M = (int32_t)M;
    p.N = (int32_t)N;
    p.K = (int32_t)K;
    p.np = 1;
    p.kper = kper16(K);
    p.pad_n = (int32_t)pad_n;
    p.alpha = alpha;
    p.beta = beta;
    return p;
}

// The sum over three pieces of one operand (hi, mid, lo of an fp32 matrix,
// `ps` elements apart) against the same other operand, in one accumulation
// chain: A = pieces (a_pieces) or B = pieces.
Gemm16Prob g16_pieced(const void* A, int64_t lda, const void* B, int64_t ldb, void* C, int64_t ldc, int64_t M,
                      int64_t N, int64_t K, bool a_pieces, int64_t ps) {
    Gemm16Prob p = g16(A, lda, B, ldb, C, ldc, M, N, K, 1.f, 0.f, N);
    p.np = 3;
    (a_pieces ? p.a_ps : p.b_ps) = ps;
    return p;
}

void set_tiles16(Gemm16Prob& p, int cfg) {
    p.tiles_m = (p.M + kGemm16Cfgs[cfg].bm - 1) / kGemm16Cfgs[cfg].bm;
    p.tiles_n = (std::max(p.N, p.pad_n) + kGemm16Cfgs[cfg].bn - 1) / kGemm16Cfgs[cfg].bn;
}

int choose_cfg16(const std::vector<Gemm16Prob>& probs) {
    int64_t t = 0;
    for (Gemm16Prob p : probs) {
        set_tiles16(p, 1);
        t += (int64_t)p.tiles_m * p.tiles_n;
    }
    return t >= kGemm16LargeMinTiles ? 1 : 0;
}

// op(A) is M x K: A stored M x K (at = false) or K x M (at = true); op(B) is
// K x N: B stored K x N (bt = false) or N x K (bt = true).
PGemm mk(bool at, bool bt, const void* A, bool a_bf16, int64_t lda, const void* B, bool b_bf16,
         int64_t ldb, float* C, int64_t ldc, int64_t M, int64_t N, int64_t K, float alpha, float beta) {
    PGemm g;
    GemmProb& p = g.p;
    p = GemmProb{};
    p.A = A;
    p.B = B;
    p.C = C;
    p.lda = lda;
    p.ldb = ldb;
    p.ldc = ldc;
    p.M = (int32_t)M;
    p.N = (int32_t)N;
    p.K = (int32_t)K;
    p.flags = vec_flags(A, lda, at ? M : K, a_bf16, B, ldb, bt ? K : N, b_bf16);
    p.alpha = alpha;
    p.beta = beta;
    set_tiles(p, 0);
    g.variant = gemm_variant(at, bt, a_bf16, b_bf16);
    return g;
}

// One grouped launch per operand variant present in the phase.
// x6: launches of a variant that has the bf16-piece mode run in it.
std::vector<GemmLaunch> put_gemm(Image& img, const std::vector<PGemm>& all, bool x6 = false) {
    std::vector<GemmLaunch> out;
    for (int v = 0; v < 16; ++v) {
        std::vector<GemmProb> probs;
        for (const PGemm& x : all)
            if (x.variant == v && x.p.tiles_m > 0 && x.p.tiles_n > 0) probs.push_back(x.p);
        if (probs.empty()) continue;
        // LPT over tiles: the cost of a tile grows with K.
        std::stable_sort(probs.begin(), probs.end(),
                         [](const GemmProb& a, const GemmProb& b) { return a.K > b.K; });
        const int cfg = choose_cfg(probs);
        std::vector<int32_t> tb;
        int total = 0;
        for (GemmProb& p : probs) {
            set_tiles(p, cfg);
            tb.push_back(total);
            total += p.tiles_m * p.tiles_n;
        }
        GemmLaunch L;
        L.variant = v | (x6 && gemm_x6_available(v) ? GV_X6 : 0);
        L.cfg = cfg;
        L.nprob = (int)probs.size();
        L.total_tiles = total;
        L.probs = img.put(probs);
        L.tb = img.put(tb);
        out.push_back(L);
    }
    return out;
}

EwLaunch put_ew(Image& img, std::vector<EwSeg> segs) {
    int64_t chunks = 0;
    for (EwSeg& s : segs) {
        s.chunk_begin = chunks;
        chunks += (s.n + kEwChunk - 1) / kEwChunk;
    }
    EwLaunch L;
    L.nseg = (int)segs.size();
    L.chunks = chunks;
    L.segs = img.put(segs);
    return L;
}

// One launch of bf16 products with one output type, LPT over tiles (the cost
// of a tile grows with K).
Gemm16Launch put_gemm16(Image& img, std::vector<Gemm16Prob> probs, bool out16) {
    Gemm16Launch L;
    L.out16 = out16;
    probs.erase(std::remove_if(probs.begin(), probs.end(),
                               [](const Gemm16Prob& p) { return p.M <= 0 || std::max(p.N, p.pad_n) <= 0; }),
                probs.end());
    if (probs.empty()) return L;
    std::stable_sort(probs.begin(), probs.end(),
                     [](const Gemm16Prob& a, const Gemm16Prob& b) { return a.np * a.K > b.np * b.K; });
    L.cfg = choose_cfg16(probs);
    std::vector<int32_t> tb;
    int total = 0;
    for (Gemm16Prob& p : probs) {
        set_tiles16(p, L.cfg);
        tb.push_back(total);
        total += p.tiles_m * p.tiles_n;
    }
    L.nprob = (int)probs.size();
    L.total_tiles = total;
    L.probs = img.put(probs);
    L.tb = img.put(tb);
    return L;
}

EwLaunch put_ew16(Image& img, std::vector<Ew16Seg> segs) {
    int64_t chunks = 0;
    for (Ew16Seg& s : segs) {
        s.chunk_begin = chunks;
        chunks += (s.n + kEwChunk - 1) / kEwChunk;
    }
    EwLaunch L;
    L.nseg = (int)segs.size();
    L.chunks = chunks;
    L.segs = img.put(segs);
    return L;
}

PackLaunch put_pack(Image& img, std::vector<PackJob> jobs) {
    int64_t chunks = 0;
    for (PackJob& j : jobs) {
        j.chunk_begin = chunks;
        chunks += (j.rows * j.ld_dst + kEwChunk - 1) / kEwChunk;
    }
    PackLaunch L;
    L.njobs = (int)jobs.size();
    L.chunks = chunks;
    L.jobs = img.put(jobs);
    return L;
}

int64_t round8(int64_t x) { return (x + 7) / 8 * 8; }

constexpr int panels(int d) { return (d + kQrPB - 1) / kQrPB; }

// Long products are split along K into chunks run as successive launches
// that accumulate into C (beta = 1 after the first chunk): each launch's fp32
// accumulation chain is then at most kChunkK / 2 MFMAs long, which keeps the
// rounding error of the refresh products and of the QR's long reductions
// near that of a blocked CPU GEMM instead of growing with the full K.
constexpr int64_t kChunkK = 1024;

// The bf16 products take up to kChunkK16 of K per launch: 16 k per MFMA, so
// the same 512-MFMA bound on an fp32 accumulation chain.
constexpr int64_t kChunkK16 = 8192;

// Appends the K chunks of a bf16 NT product (k contiguous in A and B) to
// steps[next], steps[next + 1], ...; returns the index after the last.
size_t add_k_chunked16(std::vector<std::vector<Gemm16Prob>>& steps, size_t next, const Gemm16Prob& g) {
    for (int64_t k0 = 0; k0 == 0 || k0 < g.K; k0 += kChunkK16, ++next) {
        if (steps.size() <= next) steps.resize(next + 1);
        Gemm16Prob c = g;
        c.A = g.A + k0;
        c.B = g.B + k0;
        c.K = (int32_t)std::min<int64_t>(kChunkK16, g.K - k0);
        c.kper = kper16(c.K);
        if (k0) c.beta = 1.f;
        steps[next].push_back(c);
    }
    return next;
}

// Rows of a basis per Newton-Schulz product launch: the product goes to the
// QR job's `part` buffer, which holds kNsRows rows of d floats.
constexpr int64_t kNsRows = 256;

// The K range [k0, k0 + kc) of a product, as a product of its own.
PGemm k_slice(const PGemm& g, int64_t k0, int64_t kc, float beta) {
    const bool at = g.variant & 1, bt = g.variant & 2, abf = g.variant & 4, bbf = g.variant & 8;
    const GemmProb& p = g.p;
    const char* A = (const char*)p.A + (at ? k0 * p.lda : k0) * (abf ? 2 : 4);
    const char* B = (const char*)p.B + (bt ? k0 : k0 * p.ldb) * (bbf ? 2 : 4);
    return mk(at, bt, A, abf, p.lda, B, bbf, p.ldb, p.C, p.ldc, p.M, p.N, kc, p.alpha, beta);
}

// Appends chunk c of g to steps[c] for every chunk of its K range.
void add_k_chunked(std::vector<std::vector<PGemm>>& steps, const PGemm& g) {
    const int64_t K = g.p.K;
    for (int64_t c = 0; c == 0 || c * kChunkK < K; ++c) {
        if ((int64_t)steps.size() <= c) steps.resize(c + 1);
        const int64_t k0 = c * kChunkK;
        steps[c].push_back(k_slice(g, k0, std::min(kChunkK, K - k0), c ? 1.f : g.p.beta));
    }
}



constexpr int qr_blocks(int d) { return (d + kQrNB - 1) / kQrNB; }

struct QrBytes {
    uint64_t Z, T, part, W2, Yb, Wb, W2b, Sb;
    constexpr uint64_t scratch() const { return T + part + W2 + Yb + Wb + W2b + Sb; }   // all but Z
};
constexpr QrBytes qr_job_bytes(int64_t d) {
    QrBytes b{};
    b.Z = align_up(4ull * d * d);
    b.T = align_up(4ull * panels((int)d) * kQrPB * kQrPB);
    // the in-block products' row splits (kQrMaxSplits x kQrPB rows of the
    // at most kQrPartLd in-block columns), the tall-panel path's sums, Gram
    // blocks and barrier words (qr.hip), or kNsRows rows of a Newton-Schulz
    // product, whichever is largest
    const uint64_t gmax = (uint64_t)(d + kQrTallRows - 1) / kQrTallRows;
    const uint64_t tall = gmax * (2 * kQrPB + kQrPB * kQrPB) + 256;
    const uint64_t splits = (uint64_t)kQrMaxSplits * kQrPB * kQrPartLd;
    b.part = align_up(4ull * std::max<uint64_t>(std::max<uint64_t>(splits, tall), (uint64_t)kNsRows * d));
    b.W2 = align_up(4ull * kQrPB * d);
    b.Yb = align_up(4ull * d * kQrNB);
    b.Wb = align_up(4ull * kQrNB * d);
    b.W2b = align_up(4ull * kQrNB * d);
    b.Sb = align_up(4ull * qr_blocks((int)d) * kQrNB * kQrNB);
    return b;
}

// Carve a job's scratch (everything but Z and X) from `base`; returns the
// bytes used.
uint64_t qr_assign_scratch(QrJob& j, char* base) {
    const QrBytes b = qr_job_bytes(j.d);
    uint64_t off = 0;
    j.T = (float*)(base + off); off += b.T;
    j.part = (float*)(base + off); off += b.part;
    j.W2 = (float*)(base + off); off += b.W2;
    j.Yb = (float*)(base + off); off += b.Yb;
    j.Wb = (float*)(base + off); off += b.Wb;
    j.W2b = (float*)(base + off); off += b.W2b;
    j.Sb = (float*)(base + off); off += b.Sb;
    return off;
}

// Grouped-GEMM steps of the outer QR blocks of a set of jobs. For block b
// (columns kB = b NB .. kB + w), each inner vector is one launch's problems,
// run in order:
//  fact[b]   S_b = Yb^T Yb and W = Yb^T C (C = Z[kB:, kB+w:]); the forward
//            substitution W2_q = T_q^T (W_q - S_b[q, :q] W2[:q]) panel by
//            panel; C -= Yb W2.
//  qform[b]  W = Yb^T X[kB:, kB:]; the backward substitution
//            W2_q = T_q (W_q - S_b[q, q+1:] W2[q+1:]); X[kB:, kB:] -= Yb W2.
// Yb is rebuilt from Z by qr_copy_block before each block's steps. The
// products over the L rows (S, W) run in K chunks (add_k_chunked).

struct QrSteps {
    std::vector<std::vector<std::vector<PGemm>>> fact, qform;
};

QrSteps qr_block_steps(const std::vector<QrJob>& jobs) {
    constexpr int P = kQrPanelsPerBlock;
    QrSteps S;
    int maxb = 0;
    for (const QrJob& j : jobs) maxb = std::max(maxb, qr_blocks(j.d));
    S.fact.resize(maxb);
    S.qform.resize(maxb);
    for (int b = 0; b < maxb; ++b) {
        const int64_t kB = (int64_t)b * kQrNB;
        std::vector<std::vector<PGemm>> ws, qw;
        std::vector<PGemm> upd, qupd;
        std::vector<PGemm> sub_s[P], sub_t[P], qsub_s[P], qsub_t[P];
        for (const QrJob& J : jobs) {
            const int64_t d = J.d;
            if (d <= kB) continue;
            const int64_t L = d - kB, w = std::min<int64_t>(kQrNB, L), nc = L - w;
            const int npb = (int)((w + kQrPB - 1) / kQrPB);
            float* Sb = J.Sb + b * (int64_t)kQrNB * kQrNB;
            float* Ct = J.Z + kB * d + kB + w;
            float* Cx = J.X + kB * d + kB;
            // S = Yb^T Yb, W = Yb^T C (factorisation) and W = Yb^T X[kB:, kB:] (Q formation)
            add_k_chunked(ws, mk(true, false, J.Yb, false, kQrNB, J.Yb, false, kQrNB, Sb, kQrNB, w, w, L, 1.f, 0.f));
            if (nc > 0)
                add_k_chunked(ws, mk(true, false, J.Yb, false, kQrNB, Ct, false, d, J.Wb, d, w, nc, L, 1.f, 0.f));
            // In the Q formation X[kB:, kB:] is still diag(sign R) with zeros in
            // its first w rows and columns (the later blocks, applied first,
            // touch rows and columns from kB + w only): W's first w columns
            // take only Yb's top w rows, the rest only the rows and columns
            // past kB + w.
            add_k_chunked(qw, mk(true, false, J.Yb, false, kQrNB, Cx, false, d, J.Wb, d, w, w, w, 1.f, 0.f));
            if (nc > 0)
                add_k_chunked(qw, mk(true, false, J.Yb + w * kQrNB, false, kQrNB, Cx + w * d + w, false, d, J.Wb + w,
                                     d, w, nc, nc, 1.f, 0.f));
            for (int q = 0; q < npb; ++q) {
                const int64_t r0 = (int64_t)q * kQrPB, jb = std::min<int64_t>(kQrPB, w - r0), r1 = r0 + jb;
                const float* Tq = J.T + (int64_t)(b * P + q) * kQrPB * kQrPB;
                if (nc > 0) {
                    if (q > 0)
                        sub_s[q].push_back(mk(false, false, Sb + r0 * kQrNB, false, kQrNB, J.W2b, false, d,
                                              J.Wb + r0 * d, d, jb, nc, r0, -1.f, 1.f));
                    sub_t[q].push_back(mk(true, false, Tq, false, kQrPB, J.Wb + r0 * d, false, d, J.W2b + r0 * d, d,
                                          jb, nc, jb, 1.f, 0.f));
                }
                if (q < npb - 1)
                    qsub_s[q].push_back(mk(false, false, Sb + r0 * kQrNB + r1, false, kQrNB, J.W2b + r1 * d, false, d,
                                           J.Wb + r0 * d, d, jb, L, w - r1, -1.f, 1.f));
                qsub_t[q].push_back(mk(false, false, Tq, false, kQrPB, J.Wb + r0 * d, false, d, J.W2b + r0 * d, d,
                                       jb, L, jb, 1.f, 0.f));
            }
            if (nc > 0)
                upd.push_back(mk(false, false, J.Yb, false, kQrNB, J.W2b, false, d, Ct, d, L, nc, w, -1.f, 1.f));
            qupd.push_back(mk(false, false, J.Yb, false, kQrNB, J.W2b, false, d, Cx, d, L, L, w, -1.f, 1.f));
        }
        auto add = [](std::vector<std::vector<PGemm>>& out, std::vector<PGemm>& v) {
            if (!v.empty()) out.push_back(std::move(v));
        };
        for (std::vector<PGemm>& v : ws) add(S.fact[b], v);
        for (int q = 0; q < P; ++q) {
            add(S.fact[b], sub_s[q]);
            add(S.fact[b], sub_t[q]);
        }
        add(S.fact[b], upd);
        for (std::vector<PGemm>& v : qw) add(S.qform[b], v);
        for (int q = P - 1; q >= 0; --q) {
            add(S.qform[b], qsub_s[q]);
            add(S.qform[b], qsub_t[q]);
        }
        add(S.qform[b], qupd);
    }
    return S;
}

// Refresh scratch of one matrix: Gram products B1U (n x r), B1V (m x r), the
// QR inputs ZU (m x m), ZV (n x n) and the QR scratch of both orders.
uint64_t refresh_bytes(int64_t m, int64_t n) {
    const int64_t r = std::min(m, n);
    QrBytes bu = qr_job_bytes(m), bv = qr_job_bytes(n);
    return align_up(4ull * n * r) + align_up(4ull * m * r) + bu.Z + bv.Z + bu.scratch() + bv.scratch();
}

// Refresh batches: matrices in LPT order, next-fit under the refresh cap (a
// matrix above the cap forms a batch of its own).
std::vector<std::vector<int>> plan_refresh(const opt_group_s* g, const std::vector<std::vector<int>>& plan,
                                           uint64_t overlay) {
    const uint64_t cap = refresh_capacity_of(&g->hp, overlay, state_bytes(g));
    std::vector<std::vector<int>> out;
    uint64_t used = 0;
    for (const std::vector<int>& members : plan)
        for (int mi : members) {
            const int64_t m = g->mats[mi].d.m, n = g->mats[mi].d.n;
            const uint64_t b = refresh_bytes(m, n) +
                               ((g->hp.flags & OPT_FLAG_BF16_BASES) ? align_up(4ull * m * m) + align_up(4ull * n * n) : 0);
            if (out.empty() || (used + b > cap && !out.back().empty())) {
                out.emplace_back();
                used = 0;
            }
            out.back().push_back(mi);
            used += b;
        }
    return out;
}

// Matrices whose momentum rotation takes the pieced bf16 product: fp32
// rotations without the carried rotated momentum, a bf16 M that the bf16
// GEMM reads directly (16-byte aligned), and m, n multiples of 8 (rows of M,
// M^T and the pieces are whole 16-byte groups).
bool pieced_eligible(const opt_group_s* g, const Mat& M) {
    const uint32_t off = OPT_FLAG_ROTATED_MOMENTUM | OPT_FLAG_BF16_ROTATION | OPT_FLAG_MUON |
                         OPT_FLAG_FP32_MFMA;
    return !(g->hp.flags & off) && M.bf16 && M.d.m % 8 == 0 && M.d.n % 8 == 0 && aligned(M.d.M, 16);
}

// Build every table of the group object. `region` is the device address of
// the workspace past the tables (any value when only sizes are wanted): the
// bf16 bases (bf16-rotation variant only), then the scratch.
void build(opt_group_s* g, const std::vector<std::vector<int>>& plan, char* region) {
    g->groups.clear();
    g->rbatches.clear();
    g->img.bytes.clear();
    g->scratch_bytes = 0;
    g->refresh_bytes_max = 0;
    const bool r16 = g->hp.flags & OPT_FLAG_BF16_ROTATION;
    // the tables depend on the flags, never on whether a pointer is set, so
    // that the size query (which reads no pointer) matches create
    const bool rmf = g->hp.flags & OPT_FLAG_ROTATED_MOMENTUM;
    // bases stored in 16 bits: the caller's U (V) serves as the row-padded
    // bf16 copy itself when its order is a multiple of 8
    const bool b16 = g->hp.flags & OPT_FLAG_BF16_BASES;
    g->bases_bytes = 0;
    if (r16) {
        std::vector<BasisJob> bj;
        int tiles = 0;
        for (Mat& M : g->mats) {
            const int64_t m = M.d.m, n = M.d.n, m8 = round8(m), n8 = round8(n);
            const bool own_u = b16 && m == m8, own_v = b16 && n == n8;
            char* p = region + g->bases_bytes;
            const char* p0 = p;
            if (own_u) M.Ub = (uint16_t*)M.d.U;
            else { M.Ub = (uint16_t*)p; p += align_up(2ull * m * m8); }
            M.Utb = (uint16_t*)p; p += align_up(2ull * m * m8);
            if (own_v) M.Vb = (uint16_t*)M.d.V;
            else { M.Vb = (uint16_t*)p; p += align_up(2ull * n * n8); }
            M.Vtb = (uint16_t*)p; p += align_up(2ull * n * n8);
            g->bases_bytes += (uint64_t)(p - p0);
            for (int side = 0; side < 2; ++side) {
                BasisJob j{};
                j.X = side ? (const void*)M.d.V : (const void*)M.d.U;
                j.x_bf16 = b16;
                j.Xb = (side ? own_v : own_u) ? nullptr : (side ? M.Vb : M.Ub);
                j.Xt = side ? M.Vtb : M.Utb;
                j.d = (int32_t)(side ? n : m);
                j.dp = (int32_t)round8(j.d);
                j.tile_begin = tiles;
                const int per = (j.dp + kBasisTile - 1) / kBasisTile;
                tiles += per * per;
                bj.push_back(j);
            }
        }
        g->basis_njobs = (int)bj.size();
        g->basis_tiles = tiles;
        g->basis_jobs = g->img.put(bj);
    }
    const bool muon = g->hp.flags & OPT_FLAG_MUON;
    g->transpose_njobs = g->transpose_tiles = 0;
    if (!r16 && !muon) {
        std::vector<TransposeJob> tj;
        int tiles = 0;
        for (Mat& M : g->mats) {
            const int64_t m = M.d.m;
            M.Ut = (float*)(region + g->bases_bytes);
            g->bases_bytes += align_up(4ull * m * m);
            TransposeJob j{};
            j.X = M.d.U;
            j.Xt = M.Ut;
            j.d = (int32_t)m;
            j.tile_begin = tiles;
            const int per = (int)((m + kTransposeTile - 1) / kTransposeTile);
            tiles += per * per;
            tj.push_back(j);
        }
        g->transpose_njobs = (int)tj.size();
        g->transpose_tiles = tiles;
        g->transpose_jobs = g->img.put(tj);
        std::vector<SplitJob> pj;
        int ptiles = 0;
        for (Mat& M : g->mats) {
            M.Bp = nullptr;
            if (!pieced_eligible(g, M)) continue;
            const int64_t m = M.d.m, n = M.d.n;
            M.tall = m > n;
            const int64_t d = M.tall ? m : n;
            M.Bp = (uint16_t*)(region + g->bases_bytes);
            g->bases_bytes += align_up(6ull * d * d);
            // piece p of X^T: Bp[p d^2 + c d + k] = piece_p(X[k][c])
            SplitJob j{};
            j.src = M.tall ? M.d.U : M.d.V;
            j.dst = M.Bp;
            j.ld_src = d;
            j.ld_dst = d;
            j.piece_stride = d * d;
            j.rows = j.cols = (int32_t)d;
            j.npieces = 3;
            j.src_bf16 = 0;
            j.tile_begin = ptiles;
            ptiles += (int)(((d + 31) / 32) * ((d + 31) / 32));
            pj.push_back(j);
        }
        g->pieces_njobs = (int)pj.size();
        g->pieces_tiles = ptiles;
        g->pieces_jobs = g->img.put(pj);
    }
    char* scratch = region + g->bases_bytes;
    for (const std::vector<int>& members : plan) {
        Group G;
        G.mats = members;
        if (muon) {
            // X, P (m x n) and the Gram matrix A (p x p, p = min(m, n)) per
            // matrix, then the norm partials and the inverse norms
            std::vector<MuonSeg> segs;
            std::vector<PGemm> gram, prod;
            uint64_t off = 0;
            int64_t chunks = 0;
            for (int mi : members) {
                const Mat& M = g->mats[mi];
                const opt_matrix_desc& x = M.d;
                const int64_t m = x.m, n = x.n, p = std::min(m, n), mn = m * n;
                float* X = (float*)(scratch + off); off += align_up(4ull * mn);
                float* P = (float*)(scratch + off); off += align_up(4ull * mn);
                float* A = (float*)(scratch + off); off += align_up(4ull * p * p);
                if (m >= n) {
                    gram.push_back(mk(true, false, X, false, n, X, false, n, A, n, n, n, m, 1.f, 0.f));   // X^T X
                    prod.push_back(mk(false, false, X, false, n, A, false, n, P, n, m, n, n, 1.f, 0.f));  // X A
                } else {
                    gram.push_back(mk(false, true, X, false, n, X, false, n, A, m, m, m, n, 1.f, 0.f));   // X X^T
                    prod.push_back(mk(false, false, A, false, m, X, false, n, P, n, m, n, m, 1.f, 0.f));  // A X
                }
                MuonSeg sg{};
                sg.M = x.M;
                sg.X = X;
                sg.P = P;
                sg.W = x.W;
                sg.n = mn;
                sg.chunk_begin = chunks;
                sg.m_bf16 = M.bf16;
                sg.slot = (int32_t)segs.size();
                chunks += (mn + kEwChunk - 1) / kEwChunk;
                segs.push_back(sg);
            }
            G.mu_part = (double*)(scratch + off); off += align_up(8ull * chunks);
            G.mu_inv = (float*)(scratch + off); off += align_up(4ull * segs.size());
            G.mu.nseg = (int)segs.size();
            G.mu.chunks = chunks;
            G.mu.segs = g->img.put(segs);
            // the Newton-Schulz products on bf16 MFMAs too, unless told otherwise
            const bool mx6 = !(g->hp.flags & OPT_FLAG_FP32_MFMA);
            G.mu_gram = put_gemm(g->img, gram, mx6);
            G.mu_prod = put_gemm(g->img, prod, mx6);
            std::vector<EwSeg> mom;
            for (int mi : members) {
                const Mat& M = g->mats[mi];
                EwSeg e{};
                e.a = M.d.G;
                e.b = M.d.M;
                e.n = M.d.m * M.d.n;
                e.b_bf16 = M.bf16;
                e.vec = aligned(M.d.G, 16) && aligned(M.d.M, M.bf16 ? 8 : 16);
                mom.push_back(e);
            }
            G.mom = put_ew(g->img, mom);
            G.rot_bytes = off;
            g->scratch_bytes = std::max(g->scratch_bytes, G.rot_bytes);
            g->groups.push_back(std::move(G));
            continue;
        }
        // ---- rotation scratch
        std::vector<PGemm> left, right, bl, br, right_re, left_c, right_c;
        std::vector<EwSeg> mom, adam, adam_re, adam_c;
        std::vector<Gemm16Prob> m16;
        std::vector<SplitJob> mts;
        int mt_tiles = 0;
        uint64_t off = 0;
        for (int mi : members) {
            const Mat& M = g->mats[mi];
            const opt_matrix_desc& x = M.d;
            const int64_t m = x.m, n = x.n, mn = m * n;
            float* TG = (float*)(scratch + off); off += align_up(4ull * mn);
            float* TM = (float*)(scratch + off); off += align_up(4ull * mn);
            float* Gt = (float*)(scratch + off); off += align_up(4ull * mn);
            float* mt = (float*)(scratch + off); off += align_up(4ull * mn);
            // U^T G, U^T M (A = the U^T copy, or U stored m x m read transposed)
            const bool at = !M.Ut;
            const float* UA = M.Ut ? M.Ut : x.U;
            left.push_back(mk(at, false, UA, false, m, x.G, false, n, TG, n, m, n, m, 1.f, 0.f));
            right.push_back(mk(false, false, TG, false, n, x.V, false, n, Gt, n, m, n, n, 1.f, 0.f));
            if (M.Bp && M.tall) {
                // U^T M = sum_p piece_p(U^T) M: B = M^T (bf16, n x m) in the G~ slot,
                // consumed before (U^T G) V overwrites it; then (U^T M) V
                SplitJob j{};
                j.src = x.M;
                j.dst = (uint16_t*)Gt;
                j.ld_src = n;
                j.ld_dst = m;
                j.rows = (int32_t)m;
                j.cols = (int32_t)n;
                j.npieces = 1;
                j.src_bf16 = 1;
                j.tile_begin = mt_tiles;
                mt_tiles += (int)(((m + 31) / 32) * ((n + 31) / 32));
                mts.push_back(j);
                m16.push_back(g16_pieced(M.Bp, m, Gt, m, TM, n, m, n, m, true, m * m));
                right.push_back(mk(false, false, TM, false, n, x.V, false, n, mt, n, m, n, n, 1.f, 0.f));
            } else if (M.Bp) {
                // M V = sum_p M piece_p(V^T)^T into the U^T M slot, then U^T (M V)
                m16.push_back(g16_pieced(x.M, n, M.Bp, n, TM, n, m, n, n, false, n * n));
                left.push_back(mk(at, false, UA, false, m, TM, false, n, mt, n, m, n, m, 1.f, 0.f));
            } else {
                // U^T M, then (U^T M) V
                left.push_back(mk(at, false, UA, false, m, x.M, M.bf16, n, TM, n, m, n, m, 1.f, 0.f));
                right.push_back(mk(false, false, TM, false, n, x.V, false, n, mt, n, m, n, n, 1.f, 0.f));
            }
            // U u (u in the m~ slot) -> TG slot
            bl.push_back(mk(false, false, x.U, false, m, mt, false, n, TG, n, m, n, m, 1.f, 0.f));
            // W += (-1 * lr) (U u) V^T  (B = V stored n x n read transposed)
            br.push_back(mk(false, true, TG, false, n, x.V, false, n, x.W, n, m, n, n, -1.f, 1.f));
            EwSeg e{};
            e.a = x.G;
            e.b = x.M;
            e.n = mn;
            e.b_bf16 = M.bf16;
            e.vec = aligned(x.G, 16) && aligned(x.M, M.bf16 ? 8 : 16);
            mom.push_back(e);
            EwSeg a{};
            a.a = Gt;
            a.b = mt;
            a.c = x.v;
            a.n = mn;
            a.vec = aligned(Gt, 16) && aligned(mt, 16) && aligned(x.v, 16);
            adam.push_back(a);
            if (rmf) {
                // recompute: (U^T M) V -> Mt; u = Mt / (sqrt(v) + eps) -> mt slot
                right_re.push_back(mk(false, false, TG, false, n, x.V, false, n, Gt, n, m, n, n, 1.f, 0.f));
                right_re.push_back(mk(false, false, TM, false, n, x.V, false, n, x.Mt, n, m, n, n, 1.f, 0.f));
                left_c.push_back(mk(at, false, UA, false, m, x.G, false, n, TG, n, m, n, m, 1.f, 0.f));
                right_c.push_back(mk(false, false, TG, false, n, x.V, false, n, Gt, n, m, n, n, 1.f, 0.f));
                EwSeg r = a;
                r.b = x.Mt;
                r.d = mt;
                r.vec = a.vec && aligned(x.Mt, 16);
                adam_re.push_back(r);
                r.carry = 1;
                adam_c.push_back(r);
            }
        }
        G.rot_bytes = off;
        if (r16) {
            std::vector<Gemm16Prob> s_right, s_left, s_bright, s_bleft, s_right_c, s_left_c, s_left_re;
            std::vector<Ew16Seg> m16, a16, a16_c, a16_re;
            std::vector<EwSeg> mr, ar, ar_c, ar_re;
            std::vector<PackJob> pin, pu;
            uint64_t o = 0;
            for (int mi : members) {
                const Mat& M = g->mats[mi];
                const opt_matrix_desc& x = M.d;
                const int64_t m = x.m, n = x.n, mn = m * n, m8 = round8(m), n8 = round8(n);
                const bool flat = n % 8 == 0;
                const bool m_direct = flat && M.bf16 && aligned(x.M, 16);
                uint16_t* Gb = (uint16_t*)(scratch + o); o += align_up(2ull * m * n8);   // later u
                uint16_t* Mb = m_direct ? (uint16_t*)x.M : (uint16_t*)(scratch + o);
                if (!m_direct) o += align_up(2ull * m * n8);
                uint16_t* SG = (uint16_t*)(scratch + o); o += align_up(2ull * n * m8);   // later P
                uint16_t* SM = (uint16_t*)(scratch + o); o += align_up(2ull * n * m8);
                float* Gt = (float*)(scratch + o); o += align_up(4ull * mn);
                float* mt = (float*)(scratch + o); o += align_up(4ull * mn);
                // S = (X V)^T: S[j][i] = sum_k V^T[j][k] X[i][k]   (n x m, row stride m8)
                s_right.push_back(g16(M.Vtb, n8, Gb, n8, SG, m8, n, m, n8, 1.f, 0.f, m8));
                s_right.push_back(g16(M.Vtb, n8, Mb, n8, SM, m8, n, m, n8, 1.f, 0.f, m8));
                // G~ = U^T S^T: G~[i][j] = sum_k U^T[i][k] S[j][k]  (m x n fp32)
                s_left.push_back(g16(M.Utb, m8, SG, m8, Gt, n, m, n, m8, 1.f, 0.f, n));
                s_left.push_back(g16(M.Utb, m8, SM, m8, mt, n, m, n, m8, 1.f, 0.f, n));
                if (rmf) {
                    // carried m~: G alone on carrying steps; m~ into Mt on recomputing ones
                    s_right_c.push_back(s_right[s_right.size() - 2]);
                    s_left_c.push_back(s_left[s_left.size() - 2]);
                    s_left_re.push_back(s_left[s_left.size() - 2]);
                    s_left_re.push_back(g16(M.Utb, m8, SM, m8, x.Mt, n, m, n, m8, 1.f, 0.f, n));
                }
                // P = (u V^T)^T: P[j][k] = sum_l V[j][l] u[k][l]   (n x m, into SG)
                s_bright.push_back(g16(M.Vb, n8, Gb, n8, SG, m8, n, m, n8, 1.f, 0.f, m8));
                // W -= lr U P^T: sum_k U[i][k] P[j][k]
                s_bleft.push_back(g16(M.Ub, m8, SG, m8, x.W, n, m, n, m8, -1.f, 1.f, n));
                if (flat) {
                    Ew16Seg e{};
                    e.a = x.G;
                    e.b = x.M;
                    e.o1 = Gb;
                    e.o2 = m_direct ? nullptr : Mb;
                    e.n = mn;
                    e.b_bf16 = M.bf16;
                    e.vec = aligned(x.G, 16) && aligned(x.M, M.bf16 ? 8 : 16);
                    m16.push_back(e);
                    Ew16Seg a{};
                    a.a = Gt;
                    a.b = mt;
                    a.c = x.v;
                    a.o1 = Gb;
                    a.n = mn;
                    a.vec = aligned(x.v, 16);
                    a16.push_back(a);
                    if (rmf) {
                        a.b = x.Mt;
                        a.vec = aligned(x.v, 16) && aligned(x.Mt, 16);
                        a16_re.push_back(a);
                        a.carry = 1;
                        a16_c.push_back(a);
                    }
                } else {
                    EwSeg e{};
                    e.a = x.G;
                    e.b = x.M;
                    e.n = mn;
                    e.b_bf16 = M.bf16;
                    e.vec = aligned(x.G, 16) && aligned(x.M, M.bf16 ? 8 : 16);
                    mr.push_back(e);
                    pin.push_back({x.G, Gb, m, n, n, n8, 0, 0});
                    pin.push_back({x.M, Mb, m, n, n, n8, 0, (int32_t)M.bf16});
                    EwSeg a{};
                    a.a = Gt;
                    a.b = mt;   // u over m~, then packed into Gb's buffer
                    a.c = x.v;
                    a.n = mn;
                    a.vec = aligned(x.v, 16);
                    ar.push_back(a);
                    pu.push_back({mt, Gb, m, n, n, n8, 0, 0});
                    if (rmf) {
                        a.b = x.Mt;   // u to the m~ scratch (packed from there), m~ kept in Mt
                        a.d = mt;
                        a.vec = aligned(x.v, 16) && aligned(x.Mt, 16);
                        ar_re.push_back(a);
                        a.carry = 1;
                        ar_c.push_back(a);
                    }
                }
            }
            G.r16_right.push_back(put_gemm16(g->img, s_right, true));
            G.r16_left.push_back(put_gemm16(g->img, s_left, false));
            G.r16_back_right.push_back(put_gemm16(g->img, s_bright, true));
            G.r16_back_left.push_back(put_gemm16(g->img, s_bleft, false));
            G.mom16 = put_ew16(g->img, m16);
            G.adam16 = put_ew16(g->img, a16);
            G.mom_r = put_ew(g->img, mr);
            G.adam_r = put_ew(g->img, ar);
            G.pack_in = put_pack(g->img, pin);
            G.pack_u = put_pack(g->img, pu);
            if (!s_right_c.empty()) {
                G.r16_right_c.push_back(put_gemm16(g->img, s_right_c, true));
                G.r16_left_c.push_back(put_gemm16(g->img, s_left_c, false));
                G.r16_left_re.push_back(put_gemm16(g->img, s_left_re, false));
                G.adam16_c = put_ew16(g->img, a16_c);
                G.adam16_re = put_ew16(g->img, a16_re);
                G.adam_r_c = put_ew(g->img, ar_c);
                G.adam_r_re = put_ew(g->img, ar_re);
            }
            G.rot_bytes = std::max(G.rot_bytes, o);
        }
        const bool x6 = !(g->hp.flags & OPT_FLAG_FP32_MFMA);
        G.rot_left = put_gemm(g->img, left, x6);
        G.rot_right = put_gemm(g->img, right, x6);
        if (!m16.empty()) {
            G.rot_m16.push_back(put_gemm16(g->img, m16, false));
            G.mt_nsplit = (int)mts.size();
            G.mt_tiles = mt_tiles;
            G.mt_split = g->img.put(mts);
        }
        G.back_left = put_gemm(g->img, bl, x6);
        G.back_right = put_gemm(g->img, br, x6);
        G.mom = put_ew(g->img, mom);
        G.adam = put_ew(g->img, adam);
        if (!adam_c.empty()) {
            G.rot_right_re = put_gemm(g->img, right_re, x6);
            G.rot_left_c = put_gemm(g->img, left_c, x6);
            G.rot_right_c = put_gemm(g->img, right_c, x6);
            G.adam_re = put_ew(g->img, adam_re);
            G.adam_c = put_ew(g->img, adam_c);
        }
        g->scratch_bytes = std::max(g->scratch_bytes, G.rot_bytes);
        g->groups.push_back(std::move(G));
    }

    // the refresh's Gram products and QR block updates on bf16 MFMAs too
    const bool rx6 = !(g->hp.flags & OPT_FLAG_FP32_MFMA);
    // A refresh batch's buffers start at the copies of the bases: a refresh
    // makes the copies stale (they are rebuilt from the new U, V before any
    // rotation reads them) and runs between the steps' use of the scratch.
    char* const rscratch = region;
    const uint64_t overlay = g->bases_bytes + g->scratch_bytes;
    for (const std::vector<int>& members : muon ? std::vector<std::vector<int>>{} : plan_refresh(g, plan, overlay)) {
        RefreshBatch R;
        R.mats = members;
        uint64_t off = 0;
        std::vector<PGemm> p1, p2;
        std::vector<CopyJob> comp;
        std::vector<CvtJob> widen, round16;
        int64_t widen_chunks = 0, round_chunks = 0;
        struct JobSrc { int64_t d; float* Z; float* X; int mat; int side; };
        std::vector<JobSrc> jsrc;
        for (int mi : members) {
            const Mat& M = g->mats[mi];
            opt_matrix_desc x = M.d;
            const int64_t m = x.m, n = x.n, r = std::min(m, n);
            float* B1U = (float*)(rscratch + off); off += align_up(4ull * n * r);
            float* B1V = (float*)(rscratch + off); off += align_up(4ull * m * r);
            float* ZU = (float*)(rscratch + off); off += align_up(4ull * m * m);
            float* ZV = (float*)(rscratch + off); off += align_up(4ull * n * n);
            if (b16) {
                // bases stored in 16 bits: the refresh works on fp32 copies in
                // its scratch, widened from U, V before the first pass and
                // rounded back into them after the last
                float* XU = (float*)(rscratch + off); off += align_up(4ull * m * m);
                float* XV = (float*)(rscratch + off); off += align_up(4ull * n * n);
                for (int side = 0; side < 2; ++side) {
                    const int64_t nel = side ? n * n : m * m;
                    void* b = side ? (void*)x.V : (void*)x.U;
                    float* f = side ? XV : XU;
                    widen.push_back({b, f, nel, widen_chunks, 0});
                    widen_chunks += (nel + kEwChunk - 1) / kEwChunk;
                    round16.push_back({f, b, nel, round_chunks, 1});
                    round_chunks += (nel + kEwChunk - 1) / kEwChunk;
                }
                x.U = XU;
                x.V = XV;
            }
            // B1U = M^T U[:, :r]   (n x r): A = M stored m x n read transposed
            p1.push_back(mk(true, false, x.M, M.bf16, n, x.U, false, m, B1U, r, n, r, m, 1.f, 0.f));
            // B1V = M V[:, :r]     (m x r)
            p1.push_back(mk(false, false, x.M, M.bf16, n, x.V, false, n, B1V, r, m, r, n, 1.f, 0.f));
            // ZU[:, :r] = M B1U     (m x r)
            p2.push_back(mk(false, false, x.M, M.bf16, n, B1U, false, r, ZU, m, m, r, n, 1.f, 0.f));
            // ZV[:, :r] = M^T B1V   (n x r)
            p2.push_back(mk(true, false, x.M, M.bf16, n, B1V, false, r, ZV, n, n, r, m, 1.f, 0.f));
            if (r < m) comp.push_back({x.U, ZU, (int32_t)m, (int32_t)r});
            if (r < n) comp.push_back({x.V, ZV, (int32_t)n, (int32_t)r});
            jsrc.push_back({m, ZU, x.U, M.idx, 0});
            jsrc.push_back({n, ZV, x.V, M.idx, 1});
        }
        std::stable_sort(jsrc.begin(), jsrc.end(), [](const JobSrc& a, const JobSrc& b) { return a.d > b.d; });
        std::vector<QrJob> jobs;
        std::vector<DriftJob> drift;
        for (const JobSrc& js : jsrc) drift.push_back({js.Z, (int32_t)js.d, js.mat, js.side});
        for (const JobSrc& js : jsrc) {
            QrJob j{};
            j.Z = js.Z;
            j.X = js.X;
            j.d = (int32_t)js.d;
            j.np = panels((int)js.d);
            off += qr_assign_scratch(j, rscratch + off);
            jobs.push_back(j);
            R.qr.np.push_back(j.np);
            R.qr.d.push_back(j.d);
        }
        R.ref_bytes = off;
        {
            std::vector<std::vector<PGemm>> s1, s2;
            for (const PGemm& x : p1) add_k_chunked(s1, x);
            for (const PGemm& x : p2) add_k_chunked(s2, x);
            for (const std::vector<PGemm>& st : s1) R.prod1.push_back(put_gemm(g->img, st, rx6));
            for (const std::vector<PGemm>& st : s2) R.prod2.push_back(put_gemm(g->img, st, rx6));
        }
        R.nwiden = (int)widen.size();
        R.widen_chunks = widen_chunks;
        R.widen = g->img.put(widen);
        R.round_chunks = round_chunks;
        R.round16 = g->img.put(round16);
        R.comp.n = (int)comp.size();
        R.comp.max_d = 0;
        for (const CopyJob& c : comp) R.comp.max_d = std::max(R.comp.max_d, (int)c.d);
        R.comp.jobs = g->img.put(comp);
        R.qr.njobs = (int)jobs.size();
        R.qr.max_d = jobs.empty() ? 0 : jobs[0].d;
        R.qr.jobs = g->img.put(jobs);
        {
            const QrSteps st = qr_block_steps(jobs);
            auto put_steps = [&](const std::vector<std::vector<std::vector<PGemm>>>& in,
                                 std::vector<std::vector<std::vector<GemmLaunch>>>& out) {
                out.resize(in.size());
                for (size_t b = 0; b < in.size(); ++b)
                    for (const std::vector<PGemm>& step : in[b]) out[b].push_back(put_gemm(g->img, step, rx6));
            };
            put_steps(st.fact, R.qr.fact);
            put_steps(st.qform, R.qr.qform);
        }
        // state checks and Newton-Schulz steps on the same buffers: G = X^T X
        // in Z, P = X[rows] G in the job's part buffer (kNsRows x d)
        {
            std::vector<std::vector<PGemm>> gram;
            int64_t max_d = 0;
            for (const QrJob& j : jobs) {
                const int64_t d = j.d;
                max_d = std::max(max_d, d);
                add_k_chunked(gram, mk(true, false, j.X, false, d, j.X, false, d, j.Z, d, d, d, d, 1.f, 0.f));
            }
            for (const std::vector<PGemm>& st : gram) R.gram.push_back(put_gemm(g->img, st));
            R.ndrift = (int)drift.size();
            R.drift_max_d = (int)max_d;
            R.drift_jobs = g->img.put(drift);
            for (int64_t r0 = 0; r0 < max_d; r0 += kNsRows) {
                std::vector<std::vector<PGemm>> prod;
                std::vector<NsJob> nj;
                NsChunk C;
                for (const QrJob& j : jobs) {
                    const int64_t d = j.d;
                    if (d <= r0) continue;
                    const int64_t rows = std::min<int64_t>(kNsRows, d - r0);
                    add_k_chunked(prod, mk(false, false, j.X + r0 * d, false, d, j.Z, false, d, j.part, d, rows, d, d,
                                           1.f, 0.f));
                    nj.push_back({j.X + r0 * d, j.part, rows * d});
                    C.max_n = std::max(C.max_n, rows * d);
                }
                for (const std::vector<PGemm>& st : prod) C.prod.push_back(put_gemm(g->img, st));
                C.njobs = (int)nj.size();
                C.jobs = g->img.put(nj);
                R.ns.push_back(std::move(C));
            }
        }
        g->refresh_bytes_max = std::max(g->refresh_bytes_max, R.ref_bytes);
        g->rbatches.push_back(std::move(R));
    }
    // state checks: every matrix, input order
    if (!muon) {
        std::vector<HealthSeg> hs;
        int64_t chunks = 0;
        for (const Mat& M : g->mats) {
            HealthSeg h{};
            h.W = M.d.W;
            h.M = M.d.M;
            h.v = M.d.v;
            h.n = M.d.m * M.d.n;
            h.chunk_begin = chunks;
            h.m_bf16 = M.bf16;
            h.out = M.idx;
            chunks += (h.n + kEwChunk - 1) / kEwChunk;
            hs.push_back(h);
        }
        g->health_nseg = (int)hs.size();
        g->health_chunks = chunks;
        g->health_segs = g->img.put(hs);
        g->health_out = g->img.put(std::vector<HealthOut>(g->mats.size()));
        g->scratch_bytes = std::max(g->scratch_bytes, align_up(sizeof(HealthPartial) * (uint64_t)chunks));
    }
    g->table_bytes = align_up(g->img.bytes.size());
}

// ------------------------------------------------------------- execution ----

template <class T>
const T* dptr(const opt_group_s* g, uint64_t off) {
    return (const T*)(g->ws + off);
}

hipEvent_t next_event(opt_group_s* g) {
    if (g->pool_used == g->pool.size()) {
        g->timing_overflow = true;
        return nullptr;
    }
    return g->pool[g->pool_used++];
}

// Steps whose scopes the event pool holds between two reads of the timing.
constexpr int kTimingSteps = 64;

// Upper bound on the phase scopes of one step (or one refresh_basis): the
// momentum, the four rotation phases, the Adam phase and the pieced product
// of every micro-group, one refresh scope per refresh batch, the copies of
// the bases, plus a margin.
size_t scopes_per_step(const opt_group_s* g) {
    return 8 * g->groups.size() + 2 * g->rbatches.size() + 4;
}

// Events recorded on the step's stream around every launch sequence of a
// phase; `kernels` counts the kernels the scope launched (a phase may need
// one launch per operand variant), so per-launch averages can be formed.
struct PhaseScope {
    opt_group_s* g;
    int phase;
    hipStream_t s;
    int group;
    hipEvent_t b = nullptr;
    PhaseScope(opt_group_s* g_, int ph, hipStream_t s_, int group_ = -1) : g(g_), phase(ph), s(s_), group(group_) {
        g->kernels_in_scope = 0;
        if (g->timing) {
            b = next_event(g);
            if (b) (void)hipEventRecord(b, s);
        }
    }
    ~PhaseScope() {
        if (g->timing && b) {
            hipEvent_t e = next_event(g);
            if (e) {
                (void)hipEventRecord(e, s);
                if (g->recs.size() < g->recs.capacity()) g->recs.push_back({phase, group, b, e, g->kernels_in_scope});
                else g->timing_overflow = true;
            }
        }
    }
};

hipError_t run_gemm(opt_group_s* g, const std::vector<GemmLaunch>& Ls, float alpha_scale,
                    hipStream_t s) {
    for (const GemmLaunch& L : Ls) {
        hipError_t e = launch_gemm_grouped(L.variant, L.cfg, dptr<GemmProb>(g, L.probs), dptr<int32_t>(g, L.tb),
                                           L.nprob, L.total_tiles, alpha_scale, s);
        if (e != hipSuccess) return e;
        g->kernels_in_scope += 1;
    }
    return hipSuccess;
}

hipError_t run_gemm16(opt_group_s* g, const std::vector<Gemm16Launch>& Ls, float alpha_scale, hipStream_t s) {
    for (const Gemm16Launch& L : Ls) {
        if (L.nprob == 0) continue;
        hipError_t e = launch_gemm16_grouped(L.out16, L.cfg, dptr<Gemm16Prob>(g, L.probs), dptr<int32_t>(g, L.tb),
                                             L.nprob, L.total_tiles, alpha_scale, s);
        if (e != hipSuccess) return e;
        g->kernels_in_scope += 1;
    }
    return hipSuccess;
}

hipError_t run_pack(opt_group_s* g, const PackLaunch& L, hipStream_t s) {
    if (L.njobs == 0) return hipSuccess;
    g->kernels_in_scope += 1;
    return launch_pack16(dptr<PackJob>(g, L.jobs), L.njobs, L.chunks, s);
}

// Runs of equal order among the jobs still active at panel p, in chunks of
// at most kQrMaxClasses (one launch per chunk).
std::vector<QrClasses> active_classes(const std::vector<int>& d, int p) {
    std::vector<QrClasses> out;
    QrClasses cur{};
    for (size_t i = 0; i < d.size();) {
        if (d[i] <= p * kQrPB) break;
        size_t j = i;
        while (j < d.size() && d[j] == d[i]) ++j;
        if (cur.n == kQrMaxClasses) {
            out.push_back(cur);
            cur = QrClasses{};
        }
        cur.d[cur.n] = d[i];
        cur.first[cur.n] = (int32_t)i;
        cur.count[cur.n] = (int32_t)(j - i);
        cur.n += 1;
        i = j;
    }
    if (cur.n) out.push_back(cur);
    return out;
}

// Panel p on the tall path (rows spread over resident workgroups, one
// cooperative launch) when its tallest panel has more than kTallMinRows rows
// and all its panels together at most kTallMaxRows (and the workgroups fit
// on the device): a few tall panels, which one workgroup each would
// factorise with most of the GPU idle. With many panels in flight the
// one-workgroup kernel already fills the GPU. Measured on one matrix, the
// tall path takes 0.58x the time at order 12288, 1.05x at 6144 and 1.3x at
// 3072, hence the threshold.
#ifndef MATOPT_TALL_MIN_ROWS
#define MATOPT_TALL_MIN_ROWS 6144
#endif
constexpr int kTallMinRows = MATOPT_TALL_MIN_ROWS;
constexpr int64_t kTallMaxRows = 96 * 1024;
bool use_tall_panels(const std::vector<int>& d, int p) {
    int64_t rows = 0;
    int tallest = 0;
    for (int x : d) {
        const int L = x - p * kQrPB;
        if (L <= 0) break;
        rows += L;
        tallest = std::max(tallest, L);
    }
    return tallest > kTallMinRows && rows <= kTallMaxRows;
}

// `block_steps(b, qform)` runs the grouped-GEMM steps of outer block b.
template <class BlockSteps>
hipError_t run_qr(const QrJob* jobs, const std::vector<int>& np, const std::vector<int>& d, hipStream_t s,
                  BlockSteps&& block_steps) {
    const int njobs = (int)np.size();
    if (njobs == 0) return hipSuccess;
    const int maxp = np[0], max_d = d[0];
    const int maxb = (max_d + kQrNB - 1) / kQrNB;
    hipError_t e;
    auto active_p = [&](int p) {
        int a = 0;
        while (a < njobs && np[a] > p) ++a;
        return a;
    };
    auto active_b = [&](int b) {
        int a = 0;
        while (a < njobs && d[a] > b * kQrNB) ++a;
        return a;
    };
    for (int b = 0; b < maxb; ++b) {
        for (int q = 0; q < kQrPanelsPerBlock; ++q) {
            const int p = b * kQrPanelsPerBlock + q;
            if (p >= maxp) break;
            const std::vector<QrClasses> cls = active_classes(d, p);
            if (use_tall_panels(d, p) && qr_tall_blocks(cls, p) > 0 && qr_tall_blocks(cls, p) <= qr_coop_capacity()) {
                if ((e = launch_qr_panel_tall(jobs, active_p(p), cls, p, max_d, s))) return e;
            } else if ((e = launch_qr_panel(jobs, active_p(p), p, max_d, s))) {
                return e;
            }
            for (const QrClasses& C : active_classes(d, p)) {
                if ((e = launch_qr_dots(jobs, C, p, s))) return e;
                if ((e = launch_qr_reduce(jobs, C, p, s))) return e;
                if ((e = launch_qr_update(jobs, C, p, s))) return e;
            }
        }
        if ((e = launch_qr_copy_block(jobs, active_b(b), b, max_d, s))) return e;
        if ((e = block_steps(b, false))) return e;
    }
    if ((e = launch_qr_init_q(jobs, njobs, max_d, s))) return e;
    for (int b = maxb - 1; b >= 0; --b) {
        if ((e = launch_qr_copy_block(jobs, active_b(b), b, max_d, s))) return e;
        if ((e = block_steps(b, true))) return e;
    }
    return hipSuccess;
}

hipError_t run_refresh(opt_group_s* g, const RefreshBatch& G, int power_iters, hipStream_t s) {
    PhaseScope ps(g, OPT_PHASE_REFRESH, s);
    hipError_t e;
    if (G.nwiden && (e = launch_cvt16(dptr<CvtJob>(g, G.widen), G.nwiden, G.widen_chunks, s))) return e;
    for (int it = 0; it < power_iters; ++it) {
        for (const std::vector<GemmLaunch>& st : G.prod1)
            if ((e = run_gemm(g, st, 1.f, s))) return e;
        for (const std::vector<GemmLaunch>& st : G.prod2)
            if ((e = run_gemm(g, st, 1.f, s))) return e;
        if ((e = launch_copy_cols(dptr<CopyJob>(g, G.comp.jobs), G.comp.n, G.comp.max_d, s))) return e;
        auto steps = [&](int b, bool qform) -> hipError_t {
            for (const std::vector<GemmLaunch>& st : (qform ? G.qr.qform : G.qr.fact)[b])
                if (hipError_t e2 = run_gemm(g, st, 1.f, s)) return e2;
            return hipSuccess;
        };
        if ((e = run_qr(dptr<QrJob>(g, G.qr.jobs), G.qr.np, G.qr.d, s, steps))) return e;
    }
    if (G.nwiden && (e = launch_cvt16(dptr<CvtJob>(g, G.round16), G.nwiden, G.round_chunks, s))) return e;
    return hipSuccess;
}

opt_status check_group(opt_group_t g) {
    if (!g) return fail(OPT_EINVAL, "group is NULL");
    return OPT_OK;
}

opt_status set_device(opt_group_t g) {
    int cur = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (cur != g->device) return fail(OPT_ESTATE, "group was created on device %d, current device is %d",
                                      g->device, cur);
    return OPT_OK;
}

}  // namespace

// =================================================================== ABI ====

extern "C" {

const char* opt_last_error(void) { return g_err.c_str(); }

opt_status opt_plan(const opt_matrix_desc* descs, int32_t count, const opt_hparams* hp,
                    int32_t* order, int32_t* group_of, int32_t* num_groups) {
    opt_status st = check_descs(descs, count, hp, false);
    if (st) return st;
    std::vector<int> ord;
    std::vector<std::vector<int>> groups;
    plan_groups(descs, count, hp, ord, groups);
    if (order)
        for (int k = 0; k < count; ++k) order[k] = ord[k];
    if (group_of)
        for (size_t gi = 0; gi < groups.size(); ++gi)
            for (int i : groups[gi]) group_of[i] = (int32_t)gi;
    if (num_groups) *num_groups = (int32_t)groups.size();
    return OPT_OK;
}

opt_status opt_group_workspace_parts(const opt_matrix_desc* descs, int32_t count,
                                     const opt_hparams* hp, uint64_t* parts) {
    if (!parts) return fail(OPT_EINVAL, "parts is NULL");
    opt_status st = check_descs(descs, count, hp, false);
    if (st) return st;
    std::vector<int> ord;
    std::vector<std::vector<int>> plan;
    plan_groups(descs, count, hp, ord, plan);
    opt_group_s tmp;
    tmp.hp = *hp;
    // The tables are built and thrown away: tensor pointers the caller has
    // not set yet get a stand-in address (256-byte aligned, like a real
    // allocation, and never dereferenced) so that no address arithmetic
    // starts from a null pointer.
    const uintptr_t stand_in = kAlign << 4;
    auto or_stand_in = [&](auto* p) { return p ? p : (decltype(p))stand_in; };
    for (int i = 0; i < count; ++i) {
        opt_matrix_desc x = descs[i];
        x.W = or_stand_in(x.W);
        x.G = or_stand_in(x.G);
        x.M = or_stand_in(x.M);
        if (!(hp->flags & OPT_FLAG_MUON)) {
            x.v = or_stand_in(x.v);
            x.U = or_stand_in(x.U);
            x.V = or_stand_in(x.V);
        }
        if (hp->flags & OPT_FLAG_ROTATED_MOMENTUM) x.Mt = or_stand_in(x.Mt);
        Mat M{x, i, 0.0, x.M_dtype == OPT_BF16};
        tmp.mats.push_back(M);
    }
    build(&tmp, plan, (char*)(uintptr_t)kAlign);
    parts[0] = tmp.table_bytes;
    parts[1] = tmp.bases_bytes;
    parts[2] = tmp.scratch_bytes;
    parts[3] = tmp.refresh_bytes_max;
    return OPT_OK;
}

opt_status opt_group_workspace_size(const opt_matrix_desc* descs, int32_t count,
                                    const opt_hparams* hp, uint64_t* bytes) {
    if (!bytes) return fail(OPT_EINVAL, "bytes is NULL");
    uint64_t parts[4];
    const opt_status st = opt_group_workspace_parts(descs, count, hp, parts);
    if (st) return st;
    *bytes = parts[0] + std::max(parts[1] + parts[2], parts[3]);
    return OPT_OK;
}

opt_status opt_group_create(const opt_matrix_desc* descs, int32_t count, const opt_hparams* hp,
                            void* workspace, uint64_t workspace_bytes, void* stream,
                            opt_group_t* out) {
    if (!out) return fail(OPT_EINVAL, "out is NULL");
    *out = nullptr;
    std::vector<Span> spans;
    opt_status st = check_descs(descs, count, hp, true, &spans);
    if (st) return st;
    if (!workspace) return fail(OPT_EINVAL, "workspace is NULL");
    if (!aligned(workspace, kAlign)) return fail(OPT_EINVAL, "workspace must be 256-byte aligned");
    uint64_t need = 0;
    if ((st = opt_group_workspace_size(descs, count, hp, &need))) return st;
    if (workspace_bytes < need)
        return fail(OPT_ENOWS, "workspace has %llu bytes, %llu needed",
                    (unsigned long long)workspace_bytes, (unsigned long long)need);
    {
        // every tensor's whole byte range against the part of the workspace
        // the group uses
        const uintptr_t lo = (uintptr_t)workspace, hi = lo + need;
        for (const Span& sp : spans)
            if (sp.lo < hi && lo < sp.hi)
                return fail(OPT_EINVAL, "matrix %d: %s overlaps the workspace", sp.mat, sp.what);
    }
    opt_group_s* g = new opt_group_s();
    g->hp = *hp;
    if (!g->hp.capacity_bytes) g->hp.capacity_bytes = 1ull << 29;
    for (int i = 0; i < count; ++i) {
        Mat M{descs[i], i, (double)descs[i].m * descs[i].n * (descs[i].m + descs[i].n),
              descs[i].M_dtype == OPT_BF16};
        g->mats.push_back(M);
    }
    std::vector<int> ord;
    std::vector<std::vector<int>> plan;
    plan_groups(descs, count, hp, ord, plan);
    g->ws = (char*)workspace;
    g->ws_bytes = workspace_bytes;
    // Two passes: the table size does not depend on the scratch address.
    build(g, plan, (char*)(uintptr_t)kAlign);
    const uint64_t tbytes = g->table_bytes;
    build(g, plan, g->ws + tbytes);
    if (g->table_bytes != tbytes) {
        delete g;
        return fail(OPT_ESTATE, "internal: table layout changed between passes");
    }
    hipError_t e = hipGetDevice(&g->device);
    if (e != hipSuccess) {
        delete g;
        return hip_fail(e, "hipGetDevice");
    }
    if (!g->img.bytes.empty()) {
        e = hipMemcpyAsync(g->ws, g->img.bytes.data(), g->img.bytes.size(), hipMemcpyHostToDevice,
                           (hipStream_t)stream);
        if (e != hipSuccess) {
            delete g;
            return hip_fail(e, "hipMemcpyAsync(work lists)");
        }
    }
    *out = g;
    return OPT_OK;
}

opt_status opt_group_step(opt_group_t g, void* stream) {
    opt_status st = check_group(g);
    if (st || (st = set_device(g))) return st;
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e, "pending HIP error before step");
    hipStream_t s = (hipStream_t)stream;
    g->t += 1;
    if (g->hp.flags & OPT_FLAG_MUON) {
        // orthogonalised momentum: M, then per group X_0 = M / ||M||_F and
        // ns_iters Newton-Schulz steps, the last one fused with the update
        for (const Group& G : g->groups) {
        const int gi = (int)(&G - g->groups.data());
            PhaseScope ps(g, OPT_PHASE_MOMENTUM, s, gi);
            e = launch_momentum(dptr<EwSeg>(g, G.mom.segs), G.mom.nseg, G.mom.chunks, g->hp.beta1, s);
            if (e) return hip_fail(e, "momentum launch");
            g->kernels_in_scope += G.mom.nseg > 0;
        }
        for (const Group& G : g->groups) {
        const int gi = (int)(&G - g->groups.data());
            PhaseScope ps(g, OPT_PHASE_ORTHO, s, gi);
            const MuonSeg* segs = dptr<MuonSeg>(g, G.mu.segs);
            e = launch_muon_norm(segs, G.mu.nseg, G.mu.chunks, G.mu_part, G.mu_inv, s);
            if (!e) e = launch_muon_scale(segs, G.mu.nseg, G.mu.chunks, G.mu_inv, s);
            if (e) return hip_fail(e, "orthogonalisation launch");
            g->kernels_in_scope += 3;
            for (int it = 0; it < g->hp.ns_iters; ++it) {
                if ((e = run_gemm(g, G.mu_gram, 1.f, s))) return hip_fail(e, "Newton-Schulz Gram launch");
                if ((e = run_gemm(g, G.mu_prod, 1.f, s))) return hip_fail(e, "Newton-Schulz product launch");
                const bool last = it + 1 == g->hp.ns_iters;
                if ((e = launch_muon_combine(segs, G.mu.nseg, G.mu.chunks, last, g->hp.lr, s)))
                    return hip_fail(e, "Newton-Schulz combine launch");
                g->kernels_in_scope += 1;
            }
        }
        return OPT_OK;
    }
    const bool refresh = g->hp.K > 0 && (g->t - 1) % g->hp.K == 0;
    // bf16 rotations from the second step on (the first, with v = 0, in
    // fp32), or from the first with bases stored in 16 bits (no fp32 copy)
    if ((g->hp.flags & OPT_FLAG_BF16_ROTATION) && (g->t > 1 || (g->hp.flags & OPT_FLAG_BF16_BASES))) {
        const bool carry_mode = g->hp.flags & OPT_FLAG_ROTATED_MOMENTUM;
        const bool carry = carry_mode && g->mt_valid && !refresh;
        // The bf16 copies of G and M live in the scratch that the refresh and
        // every micro-group share, so each group makes its own right before
        // its rotations: with the momentum update on steps without a refresh,
        // after the refresh (which must see the updated M) otherwise.
        if (refresh) {
            for (const Group& G : g->groups) {
        const int gi = (int)(&G - g->groups.data());
                PhaseScope ps(g, OPT_PHASE_MOMENTUM, s, gi);
                e = launch_momentum(dptr<EwSeg>(g, G.mom.segs), G.mom.nseg, G.mom.chunks, g->hp.beta1, s);
                if (e) return hip_fail(e, "momentum launch");
                g->kernels_in_scope += G.mom.nseg > 0;
            }
            for (const RefreshBatch& R : g->rbatches)
                if ((e = run_refresh(g, R, g->hp.power_iters, s))) return hip_fail(e, "refresh launch");
            g->copies_valid = false;
        }
        if (!g->copies_valid) {
            PhaseScope ps(g, OPT_PHASE_REFRESH, s);
            if ((e = launch_basis16(dptr<BasisJob>(g, g->basis_jobs), g->basis_njobs, g->basis_tiles, s)))
                return hip_fail(e, "basis conversion launch");
            g->kernels_in_scope += 1;
            g->copies_valid = true;
        }
        for (const Group& G : g->groups) {
        const int gi = (int)(&G - g->groups.data());
            {
                PhaseScope ps(g, OPT_PHASE_MOMENTUM, s, gi);
                if (refresh) {
                    e = launch_convert16(dptr<Ew16Seg>(g, G.mom16.segs), G.mom16.nseg, G.mom16.chunks, s);
                    g->kernels_in_scope += G.mom16.nseg > 0;
                } else {
                    e = launch_momentum16(dptr<Ew16Seg>(g, G.mom16.segs), G.mom16.nseg, G.mom16.chunks, g->hp.beta1,
                                          s);
                    if (!e)
                        e = launch_momentum(dptr<EwSeg>(g, G.mom_r.segs), G.mom_r.nseg, G.mom_r.chunks, g->hp.beta1,
                                            s);
                    g->kernels_in_scope += (G.mom16.nseg > 0) + (G.mom_r.nseg > 0);
                }
                if (!e) e = run_pack(g, G.pack_in, s);
                if (e) return hip_fail(e, "momentum launch");
            }
            {
                PhaseScope ps(g, OPT_PHASE_ROT_RIGHT, s, gi);
                if ((e = run_gemm16(g, carry ? G.r16_right_c : G.r16_right, 1.f, s)))
                    return hip_fail(e, "rotation launch");
            }
            {
                PhaseScope ps(g, OPT_PHASE_ROT_LEFT, s, gi);
                const std::vector<Gemm16Launch>& L = !carry_mode ? G.r16_left : (carry ? G.r16_left_c : G.r16_left_re);
                if ((e = run_gemm16(g, L, 1.f, s))) return hip_fail(e, "rotation launch");
            }
            {
                PhaseScope ps(g, OPT_PHASE_ADAM, s, gi);
                const EwLaunch& A16 = !carry_mode ? G.adam16 : (carry ? G.adam16_c : G.adam16_re);
                const EwLaunch& AR = !carry_mode ? G.adam_r : (carry ? G.adam_r_c : G.adam_r_re);
                e = launch_adam16(dptr<Ew16Seg>(g, A16.segs), A16.nseg, A16.chunks, g->hp.beta1, g->hp.beta2,
                                  g->hp.eps, s);
                if (!e)
                    e = launch_rotated_adam(dptr<EwSeg>(g, AR.segs), AR.nseg, AR.chunks, g->hp.beta1, g->hp.beta2,
                                            g->hp.eps, s);
                if (!e) e = run_pack(g, G.pack_u, s);
                if (e) return hip_fail(e, "rotated Adam launch");
                g->kernels_in_scope += (A16.nseg > 0) + (AR.nseg > 0);
            }
            {
                PhaseScope ps(g, OPT_PHASE_BACK_RIGHT, s, gi);
                if ((e = run_gemm16(g, G.r16_back_right, 1.f, s))) return hip_fail(e, "rotation launch");
            }
            {
                PhaseScope ps(g, OPT_PHASE_BACK_LEFT, s, gi);
                if ((e = run_gemm16(g, G.r16_back_left, g->hp.lr, s))) return hip_fail(e, "update launch");
            }
        }
        g->mt_valid = carry_mode;
        return OPT_OK;
    }
    // Momentum of every group first: a refresh must see the updated M.
    for (const Group& G : g->groups) {
        const int gi = (int)(&G - g->groups.data());
        PhaseScope ps(g, OPT_PHASE_MOMENTUM, s, gi);
        e = launch_momentum(dptr<EwSeg>(g, G.mom.segs), G.mom.nseg, G.mom.chunks, g->hp.beta1, s);
        if (e) return hip_fail(e, "momentum launch");
        g->kernels_in_scope += G.mom.nseg > 0;
    }
    if (refresh) {
        for (const RefreshBatch& R : g->rbatches)
            if ((e = run_refresh(g, R, g->hp.power_iters, s))) return hip_fail(e, "refresh launch");
        g->copies_valid = false;
    }
    if (g->transpose_njobs && !g->copies_valid) {
        PhaseScope ps(g, OPT_PHASE_REFRESH, s);
        if ((e = launch_transpose32(dptr<TransposeJob>(g, g->transpose_jobs), g->transpose_njobs,
                                    g->transpose_tiles, s)))
            return hip_fail(e, "basis transpose launch");
        if (g->pieces_njobs &&
            (e = launch_split16(dptr<SplitJob>(g, g->pieces_jobs), g->pieces_njobs, g->pieces_tiles, s)))
            return hip_fail(e, "basis pieces launch");
        g->kernels_in_scope += 1 + (g->pieces_njobs > 0);
        g->copies_valid = true;
    }
    // with the carried rotated momentum: recompute m~ when the bases are new
    // to it, else carry it (G alone is rotated)
    const bool carry_mode = g->hp.flags & OPT_FLAG_ROTATED_MOMENTUM;
    const bool carry = carry_mode && g->mt_valid && !refresh;
    for (const Group& G : g->groups) {
        const int gi = (int)(&G - g->groups.data());
        if (!G.rot_m16.empty()) {
            PhaseScope ps(g, OPT_PHASE_ROT_PIECED, s, gi);
            if (G.mt_nsplit) {
                if ((e = launch_split16(dptr<SplitJob>(g, G.mt_split), G.mt_nsplit, G.mt_tiles, s)))
                    return hip_fail(e, "momentum transpose launch");
                g->kernels_in_scope += 1;
            }
            if ((e = run_gemm16(g, G.rot_m16, 1.f, s))) return hip_fail(e, "rotation launch");
        }
        {
            PhaseScope ps(g, OPT_PHASE_ROT_LEFT, s, gi);
            if ((e = run_gemm(g, carry ? G.rot_left_c : G.rot_left, 1.f, s))) return hip_fail(e, "rotation launch");
        }
        {
            PhaseScope ps(g, OPT_PHASE_ROT_RIGHT, s, gi);
            const std::vector<GemmLaunch>& L = !carry_mode ? G.rot_right : (carry ? G.rot_right_c : G.rot_right_re);
            if ((e = run_gemm(g, L, 1.f, s))) return hip_fail(e, "rotation launch");
        }
        {
            PhaseScope ps(g, OPT_PHASE_ADAM, s, gi);
            const EwLaunch& A = !carry_mode ? G.adam : (carry ? G.adam_c : G.adam_re);
            e = launch_rotated_adam(dptr<EwSeg>(g, A.segs), A.nseg, A.chunks, g->hp.beta1, g->hp.beta2, g->hp.eps,
                                    s);
            if (e) return hip_fail(e, "rotated Adam launch");
            g->kernels_in_scope += A.nseg > 0;
        }
        {
            PhaseScope ps(g, OPT_PHASE_BACK_LEFT, s, gi);
            if ((e = run_gemm(g, G.back_left, 1.f, s))) return hip_fail(e, "rotation launch");
        }
        {
            PhaseScope ps(g, OPT_PHASE_BACK_RIGHT, s, gi);
            if ((e = run_gemm(g, G.back_right, g->hp.lr, s))) return hip_fail(e, "update launch");
        }
    }
    g->mt_valid = carry_mode;
    return OPT_OK;
}

opt_status opt_group_refresh_basis(opt_group_t g, int32_t power_iters, void* stream) {
    opt_status st = check_group(g);
    if (st || (st = set_device(g))) return st;
    if (g->hp.flags & OPT_FLAG_MUON) return fail(OPT_EUNSUPPORTED, "no bases with OPT_FLAG_MUON");
    if (power_iters < 1) return fail(OPT_EINVAL, "power_iters must be >= 1");
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e, "pending HIP error before refresh");
    g->mt_valid = false;
    g->copies_valid = false;
    for (const RefreshBatch& R : g->rbatches)
        if ((e = run_refresh(g, R, power_iters, (hipStream_t)stream))) return hip_fail(e, "refresh launch");
    return OPT_OK;
}

opt_status opt_group_health(opt_group_t g, opt_health* out, void* stream) {
    opt_status st = check_group(g);
    if (st || (st = set_device(g))) return st;
    if (g->hp.flags & OPT_FLAG_MUON) return fail(OPT_EUNSUPPORTED, "no bases with OPT_FLAG_MUON");
    if (g->hp.flags & OPT_FLAG_BF16_BASES)
        return fail(OPT_EUNSUPPORTED, "state checks read fp32 bases; not with OPT_FLAG_BF16_BASES");
    if (!out) return fail(OPT_EINVAL, "out is NULL");
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e, "pending HIP error before health");
    hipStream_t s = (hipStream_t)stream;
    HealthOut* dout = (HealthOut*)(g->ws + g->health_out);
    HealthPartial* part = (HealthPartial*)(g->ws + g->table_bytes + g->bases_bytes);
    const HealthSeg* segs = dptr<HealthSeg>(g, g->health_segs);
    if ((e = launch_health_clear(dout, (int)g->mats.size(), s))) return hip_fail(e, "health launch");
    if ((e = launch_health_partials(segs, g->health_nseg, g->health_chunks, part, s))) return hip_fail(e, "health launch");
    if ((e = launch_health_final(segs, g->health_nseg, part, dout, s))) return hip_fail(e, "health launch");
    // the drift's Gram products use the refresh buffers, which overlay the
    // copies of the bases
    g->copies_valid = false;
    for (const RefreshBatch& R : g->rbatches) {
        for (const std::vector<GemmLaunch>& stp : R.gram)
            if ((e = run_gemm(g, stp, 1.f, s))) return hip_fail(e, "Gram launch");
        if ((e = launch_drift(dptr<DriftJob>(g, R.drift_jobs), R.ndrift, R.drift_max_d, dout, s)))
            return hip_fail(e, "drift launch");
    }
    std::vector<HealthOut> h(g->mats.size());
    if ((e = hipMemcpyAsync(h.data(), dout, sizeof(HealthOut) * h.size(), hipMemcpyDeviceToHost, s)))
        return hip_fail(e, "health copy");
    if ((e = hipStreamSynchronize(s))) return hip_fail(e, "health synchronise");
    for (size_t i = 0; i < h.size(); ++i) {
        const HealthOut& r = h[i];
        const double n = (double)r.n, mean = r.s / n;
        opt_health& o = out[i];
        o.orth_U = __builtin_bit_cast(float, r.drift_u);
        o.orth_V = __builtin_bit_cast(float, r.drift_v);
        o.v_mean_abs = r.sabs / n;
        o.v_std = std::sqrt(std::max(0.0, r.s2 / n - mean * mean));
        o.v_min = r.vmin;
        o.v_max = r.vmax;
        o.nonfinite = r.nonfinite;
    }
    return OPT_OK;
}

opt_status opt_group_reorthonormalize(opt_group_t g, int32_t iters, void* stream) {
    opt_status st = check_group(g);
    if (st || (st = set_device(g))) return st;
    if (g->hp.flags & OPT_FLAG_MUON) return fail(OPT_EUNSUPPORTED, "no bases with OPT_FLAG_MUON");
    if (g->hp.flags & OPT_FLAG_BF16_BASES)
        return fail(OPT_EUNSUPPORTED, "re-orthonormalisation works on fp32 bases; not with OPT_FLAG_BF16_BASES");
    if (iters < 0) return fail(OPT_EINVAL, "iters must be >= 0");
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e, "pending HIP error before re-orthonormalisation");
    hipStream_t s = (hipStream_t)stream;
    if (iters > 0) g->mt_valid = g->copies_valid = false;
    for (int it = 0; it < iters; ++it)
        for (const RefreshBatch& R : g->rbatches) {
            for (const std::vector<GemmLaunch>& stp : R.gram)
                if ((e = run_gemm(g, stp, 1.f, s))) return hip_fail(e, "Gram launch");
            for (const NsChunk& C : R.ns) {
                for (const std::vector<GemmLaunch>& stp : C.prod)
                    if ((e = run_gemm(g, stp, 1.f, s))) return hip_fail(e, "Newton-Schulz product launch");
                if ((e = launch_ns_combine(dptr<NsJob>(g, C.jobs), C.njobs, C.max_n, s)))
                    return hip_fail(e, "Newton-Schulz combine launch");
            }
        }
    return OPT_OK;
}

opt_status opt_group_get_step(opt_group_t g, int64_t* t) {
    if (opt_status st = check_group(g)) return st;
    if (!t) return fail(OPT_EINVAL, "t is NULL");
    *t = g->t;
    return OPT_OK;
}

opt_status opt_group_set_step(opt_group_t g, int64_t t) {
    if (opt_status st = check_group(g)) return st;
    if (t < 0) return fail(OPT_EINVAL, "t must be >= 0");
    g->t = t;
    g->mt_valid = false;   // a resumed job recomputes the rotated momentum
    g->copies_valid = false;   // and the copies of the bases (the caller may have written U, V)
    return OPT_OK;
}

opt_status opt_group_set_lr(opt_group_t g, float lr) {
    if (opt_status st = check_group(g)) return st;
    if (!std::isfinite(lr)) return fail(OPT_EINVAL, "lr must be finite");
    g->hp.lr = lr;
    return OPT_OK;
}

opt_status opt_group_set_timing(opt_group_t g, int32_t enable) {
    if (opt_status st = check_group(g)) return st;
    g->recs.clear();
    g->pool_used = 0;
    g->timing_overflow = false;
    for (int i = 0; i < OPT_NUM_PHASES; ++i) {
        g->acc_ms[i] = 0.0;
        g->acc_kernels[i] = 0;
    }
    g->acc_group_ms.assign(g->groups.size(), 0.0);
    g->timing = false;
    if (enable) {
        const size_t events = 2 * scopes_per_step(g) * kTimingSteps;
        if (opt_status st = set_device(g)) return st;
        while (g->pool.size() < events) {
            hipEvent_t e;
            hipError_t he = hipEventCreate(&e);
            if (he != hipSuccess) return hip_fail(he, "hipEventCreate");
            g->pool.push_back(e);
        }
        g->recs.reserve(events / 2);
        g->timing = true;
    }
    return OPT_OK;
}

namespace {
// Synchronises with the last recorded event and folds the records into the
// totals, freeing the event pool.
opt_status fold_timing(opt_group_t g) {
    g->acc_group_ms.resize(g->groups.size(), 0.0);
    if (!g->recs.empty()) {
        hipError_t e = hipEventSynchronize(g->recs.back().e);
        if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize");
        for (auto& r : g->recs) {
            float t = 0.f;
            e = hipEventElapsedTime(&t, r.b, r.e);
            if (e != hipSuccess) return hip_fail(e, "hipEventElapsedTime");
            g->acc_ms[r.phase] += t;
            g->acc_kernels[r.phase] += r.kernels;
            if (r.group >= 0) g->acc_group_ms[r.group] += t;
        }
        g->recs.clear();
    }
    g->pool_used = 0;
    if (g->timing_overflow)
        return fail(OPT_ESTATE, "timing: more phase scopes than the %d steps the event pool holds were "
                                "recorded between two reads; the totals miss some",
                    kTimingSteps);
    return OPT_OK;
}
}  // namespace

opt_status opt_group_read_timing(opt_group_t g, double* ms, int64_t* launches) {
    if (opt_status st = check_group(g)) return st;
    const opt_status st = fold_timing(g);
    if (st == OPT_EHIP) return st;
    for (int i = 0; i < OPT_NUM_PHASES; ++i) {
        if (ms) ms[i] = g->acc_ms[i];
        if (launches) launches[i] = g->acc_kernels[i];
    }
    return st;
}

opt_status opt_group_read_group_timing(opt_group_t g, double* ms, int32_t count) {
    if (opt_status st = check_group(g)) return st;
    if (!ms) return fail(OPT_EINVAL, "ms is NULL");
    if (count != (int32_t)g->groups.size())
        return fail(OPT_EINVAL, "count is %d, the group has %d micro-groups", count, (int)g->groups.size());
    const opt_status st = fold_timing(g);
    if (st == OPT_EHIP) return st;
    for (int32_t k = 0; k < count; ++k) ms[k] = g->acc_group_ms[k];
    return st;
}

void opt_group_destroy(opt_group_t g) {
    if (!g) return;
    for (hipEvent_t e : g->pool) (void)hipEventDestroy(e);
    delete g;
}

// ------------------------------------------------------- building blocks ----

namespace {
opt_status gemm_entry(bool x6, int32_t trans_a, int32_t trans_b, int64_t M, int64_t N, int64_t K, float alpha,
                      const void* A, int32_t a_dtype, int64_t lda, const void* B, int32_t b_dtype, int64_t ldb,
                      float beta, float* C, int64_t ldc, void* stream) {
    if (M < 0 || N < 0 || K < 0) return fail(OPT_EINVAL, "negative dimension");
    if (M > INT32_MAX / 2 || N > INT32_MAX / 2 || K > INT32_MAX / 2)
        return fail(OPT_EUNSUPPORTED, "dimension too large");
    if ((a_dtype != OPT_F32 && a_dtype != OPT_BF16) || (b_dtype != OPT_F32 && b_dtype != OPT_BF16))
        return fail(OPT_EUNSUPPORTED, "operand dtype must be OPT_F32 or OPT_BF16");
    if (M == 0 || N == 0) return OPT_OK;
    if (!C) return fail(OPT_EINVAL, "C is NULL");
    if (ldc < N) return fail(OPT_EINVAL, "ldc < N");
    if (K > 0) {
        if (!A || !B) return fail(OPT_EINVAL, "A or B is NULL");
        if (trans_a ? lda < M : lda < K) return fail(OPT_EINVAL, "lda too small");
        if (trans_b ? ldb < K : ldb < N) return fail(OPT_EINVAL, "ldb too small");
    }
    const PGemm pg = mk(trans_a != 0, trans_b != 0, A, a_dtype == OPT_BF16, lda, B, b_dtype == OPT_BF16, ldb,
                        C, ldc, M, N, K, alpha, beta);
    if (x6 && !gemm_x6_available(pg.variant))
        return fail(OPT_EUNSUPPORTED, "no bf16-piece product for this operand layout and dtype combination");
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e, "pending HIP error before gemm");
    GemmProb single = pg.p;
    const int cfg = choose_cfg({single});
    set_tiles(single, cfg);
    e = launch_gemm_single(pg.variant | (x6 ? GV_X6 : 0), cfg, single, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "gemm launch");
    return OPT_OK;
}
}  // namespace

opt_status opt_gemm(int32_t trans_a, int32_t trans_b, int64_t M, int64_t N, int64_t K, float alpha,
                    const void* A, int32_t a_dtype, int64_t lda, const void* B, int32_t b_dtype,
                    int64_t ldb, float beta, float* C, int64_t ldc, void* stream) {
    return gemm_entry(false, trans_a, trans_b, M, N, K, alpha, A, a_dtype, lda, B, b_dtype, ldb, beta, C, ldc,
                      stream);
}

opt_status opt_gemm_x6(int32_t trans_a, int32_t trans_b, int64_t M, int64_t N, int64_t K, float alpha,
                       const void* A, int32_t a_dtype, int64_t lda, const void* B, int32_t b_dtype,
                       int64_t ldb, float beta, float* C, int64_t ldc, void* stream) {
    return gemm_entry(true, trans_a, trans_b, M, N, K, alpha, A, a_dtype, lda, B, b_dtype, ldb, beta, C, ldc,
                      stream);
}

opt_status opt_gemm_bf16(int64_t M, int64_t N, int64_t K, float alpha, const void* A, int64_t lda,
                         const void* B, int64_t ldb, float beta, void* C, int32_t c_dtype, int64_t ldc,
                         void* stream) {
    if (M < 0 || N < 0 || K < 0) return fail(OPT_EINVAL, "negative dimension");
    if (M > INT32_MAX / 2 || N > INT32_MAX / 2 || K > INT32_MAX / 2)
        return fail(OPT_EUNSUPPORTED, "dimension too large");
    if (c_dtype != OPT_F32 && c_dtype != OPT_BF16) return fail(OPT_EUNSUPPORTED, "c_dtype must be OPT_F32 or OPT_BF16");
    if (c_dtype == OPT_BF16 && beta != 0.f) return fail(OPT_EINVAL, "a bf16 C needs beta == 0");
    if (M == 0 || N == 0) return OPT_OK;
    if (!C) return fail(OPT_EINVAL, "C is NULL");
    if (ldc < N) return fail(OPT_EINVAL, "ldc < N");
    if (!aligned(C, c_dtype == OPT_F32 ? 4 : 2)) return fail(OPT_EINVAL, "C is not aligned to its element size");
    if (K % 8) return fail(OPT_EINVAL, "K must be a multiple of 8");
    if (K > 0) {
        if (!A || !B) return fail(OPT_EINVAL, "A or B is NULL");
        if (lda < K || ldb < K) return fail(OPT_EINVAL, "lda and ldb must be >= K");
        if (lda % 8 || ldb % 8) return fail(OPT_EINVAL, "lda and ldb must be multiples of 8");
        if (!aligned(A, 16) || !aligned(B, 16)) return fail(OPT_EINVAL, "A and B must be 16-byte aligned");
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e, "pending HIP error before gemm");
    Gemm16Prob p = g16(A, lda, B, ldb, C, ldc, M, N, K, alpha, beta, N);
    const int cfg = choose_cfg16({p});
    set_tiles16(p, cfg);
    e = launch_gemm16_single(c_dtype == OPT_BF16, cfg, p, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "bf16 gemm launch");
    return OPT_OK;
}

opt_status opt_orthonormalize_workspace_size(int64_t d, uint64_t* bytes) {
    if (!bytes) return fail(OPT_EINVAL, "bytes is NULL");
    if (d < 1) return fail(OPT_EINVAL, "d must be >= 1");
    if (d > OPT_MAX_DIM) return fail(OPT_EUNSUPPORTED, "d must be <= %d", OPT_MAX_DIM);
    QrBytes b = qr_job_bytes(d);
    *bytes = align_up(sizeof(QrJob)) + b.scratch();
    return OPT_OK;
}

}  // extern "C"

namespace {
__global__ void put_job_kernel(QrJob* dst, QrJob val) { *dst = val; }
}  // namespace

namespace {
// The QR of one d x d matrix with its job record and scratch at `workspace`
// (at least opt_orthonormalize_workspace_size(d) bytes, 256-byte aligned).
opt_status orthonormalize_in(float* Z, float* Q, int64_t d, char* w, hipStream_t s) {
    const uintptr_t zl = (uintptr_t)Z, zh = zl + 4ull * d * d, ql = (uintptr_t)Q, qh = ql + 4ull * d * d;
    if (zl < qh && ql < zh) return fail(OPT_EINVAL, "Z and Q overlap");
    QrJob j{};
    j.Z = Z;
    j.X = Q;
    j.d = (int32_t)d;
    j.np = panels((int)d);
    qr_assign_scratch(j, w + align_up(sizeof(QrJob)));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e, "pending HIP error before orthonormalize");
    hipLaunchKernelGGL(put_job_kernel, dim3(1), dim3(1), 0, s, (QrJob*)w, j);
    if ((e = hipGetLastError())) return hip_fail(e, "job upload");
    std::vector<int> np{j.np}, dd{(int)d};
    // one job: every block step has one problem, passed by value; the block
    // products on bf16 MFMAs at fp32 accuracy, as in the step's refresh
    const QrSteps st = qr_block_steps({j});
    auto steps = [&](int b, bool qform) -> hipError_t {
        for (const std::vector<PGemm>& step : (qform ? st.qform : st.fact)[b])
            for (const PGemm& pg : step) {
                GemmProb p1 = pg.p;
                const int cfg = choose_cfg({p1});
                set_tiles(p1, cfg);
                const int v = pg.variant | (gemm_x6_available(pg.variant) ? GV_X6 : 0);
                if (hipError_t e2 = launch_gemm_single(v, cfg, p1, s)) return e2;
            }
        return hipSuccess;
    };
    if ((e = run_qr((const QrJob*)w, np, dd, s, steps))) return hip_fail(e, "QR launch");
    return OPT_OK;
}
}  // namespace

extern "C" opt_status opt_orthonormalize(float* Z, float* Q, int64_t d, void* workspace,
                                         uint64_t workspace_bytes, void* stream) {
    uint64_t need = 0;
    if (opt_status st = opt_orthonormalize_workspace_size(d, &need)) return st;
    if (!Z || !Q || !workspace) return fail(OPT_EINVAL, "a pointer is NULL");
    if (!aligned(workspace, kAlign)) return fail(OPT_EINVAL, "workspace must be 256-byte aligned");
    if (workspace_bytes < need) return fail(OPT_ENOWS, "workspace too small: %llu < %llu",
                                            (unsigned long long)workspace_bytes, (unsigned long long)need);
    return orthonormalize_in(Z, Q, d, (char*)workspace, (hipStream_t)stream);
}

// ------------------------------------------ the entry point that allocates nothing ----
//
// opt_orthonormalize_static keeps its QR job record and scratch in `scratch`,
// a file-scope device array sized for one job of order OPT_STATIC_MAX_DIM.
// Each GPU the library runs on holds its own copy until the process ends. In
// host code the array's name is only a host-side stand-in, so its device
// address on each device is taken once with hipGetSymbolAddress (with that
// device current) and only that address is passed to kernels.

namespace {
constexpr uint64_t kStaticScratchBytes = align_up(sizeof(QrJob)) + qr_job_bytes(OPT_STATIC_MAX_DIM).scratch();
static_assert(kStaticScratchBytes <= (40ull << 20), "the fixed scratch is meant to stay modest");

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

static __device__ __align__(256) char scratch[kStaticScratchBytes];

namespace {
// The current device's address of `scratch`, looked up on its first use there.
opt_status static_scratch(char** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices) return fail(OPT_EUNSUPPORTED, "device index %d beyond %d", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
        if (!p || !aligned(p, kAlign)) return fail(OPT_EHIP, "scratch has no aligned device address");
        g_scratch_ptr[dev] = p;
    }
    *out = (char*)g_scratch_ptr[dev];
    return OPT_OK;
}
}  // namespace

extern "C" opt_status opt_orthonormalize_static(float* Z, float* Q, int64_t d, void* stream) {
    if (d < 1) return fail(OPT_EINVAL, "d must be >= 1");
    if (d > OPT_STATIC_MAX_DIM)
        return fail(OPT_EUNSUPPORTED,
                    "d = %lld exceeds %d, the largest order the fixed scratch of opt_orthonormalize_static "
                    "holds (use opt_orthonormalize with a workspace)",
                    (long long)d, OPT_STATIC_MAX_DIM);
    if (!Z || !Q) return fail(OPT_EINVAL, "a pointer is NULL");
    static_assert(align_up(sizeof(QrJob)) + qr_job_bytes(1).scratch() <= kStaticScratchBytes, "");
    char* w = nullptr;
    if (opt_status st = static_scratch(&w)) return st;
    return orthonormalize_in(Z, Q, d, w, (hipStream_t)stream);
}
