// Internal structures shared by the host scheduler (api.hip) and the kernels.
// Everything here is device-visible plain data: the host builds arrays of
// these once per group and uploads them into the caller's workspace.
#pragma once

#include <vector>

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemm.h"   // the grouped GEMM (rotations, Gram products, QR block updates)
#include "gmem.h"
#include "matopt.h"

namespace matopt {

// Records the error text returned by opt_last_error() and passes st through.
opt_status fail(opt_status st, const char* fmt, ...);

// --------------------------------------------------------- elementwise ----

struct EwSeg {
    const float* a;       // momentum: G      rotated Adam: G~
    void* b;              // momentum: M      rotated Adam: m~ (in; u out when d is NULL)
    float* c;             // rotated Adam: v
    float* d;             // rotated Adam: u out (NULL: u overwrites m~ in b)
    int64_t n;            // elements
    int64_t chunk_begin;  // first chunk of this segment in the launch
    int32_t b_bf16;       // momentum stored as bfloat16
    int32_t vec;          // all pointers 16-byte aligned (vector path)
    int32_t carry;        // rotated Adam: first b <- beta1 b + (1 - beta1) a (the carried m~)
};

constexpr int kEwThreads = 256;
constexpr int kEwPerThread = 16;
constexpr int kEwChunk = kEwThreads * kEwPerThread;

hipError_t launch_momentum(const EwSeg* segs, int nseg, int64_t total_chunks, float beta1,
                           hipStream_t s);
hipError_t launch_rotated_adam(const EwSeg* segs, int nseg, int64_t total_chunks, float beta1, float beta2,
                               float eps, hipStream_t s);

// A d x d fp32 matrix X to its transpose Xt (both row-major, row stride d):
// 32 x 32 tiles through LDS, reads and writes along rows; tile_begin is the
// job's first tile of ceil(d / 32)^2.
struct TransposeJob {
    const float* X;
    float* Xt;
    int32_t d;
    int32_t tile_begin;
};
constexpr int kTransposeTile = 32;
hipError_t launch_transpose32(const TransposeJob* jobs, int njobs, int total_tiles, hipStream_t s);

// ------------------------------------------------------------------ QR ----

constexpr int kQrPB = 64;          // panel width (reflectors per compact-WY block)
#ifndef MATOPT_QR_PANELS_PER_BLOCK
#define MATOPT_QR_PANELS_PER_BLOCK 4
#endif
constexpr int kQrPanelsPerBlock = MATOPT_QR_PANELS_PER_BLOCK;
constexpr int kQrNB = kQrPB * kQrPanelsPerBlock;   // outer block width
constexpr int kQrPartLd = kQrNB;   // row stride of the split partials (in-block columns < kQrNB)
constexpr int kQrMaxSplits = 16;   // row splits of the in-block reflector-transpose products
constexpr int kQrReduceCols = 64;  // columns per workgroup of the split reduction
constexpr int kQrPanelThreads = 512;

// One d x d orthonormalisation: Z (row stride d) is factorised in place, Q is
// formed in X. Scratch: T (np * PB * PB: the panels' compact-WY factors),
// part (the in-block products' split partials, kQrMaxSplits * PB rows of
// kQrPartLd; also the tall-panel sums and a Newton-Schulz product's rows)
// and W2 (PB * d) for the in-block updates, and
// for the outer blocks Yb (d * NB: the block's reflectors as an explicit
// unit-lower matrix, row stride NB), Wb and W2b (NB * d each, row stride d)
// and Sb (nb * NB * NB: every block's reflector Gram matrix).
struct QrJob {
    float* Z;
    float* X;
    float* T;
    float* part;
    float* W2;
    float* Yb;
    float* Wb;
    float* W2b;
    float* Sb;
    int32_t d;
    int32_t np;   // panels: ceil(d / PB)
};

// Jobs are sorted by d descending, so the jobs still active at panel p are a
// prefix of the array; `njobs` passed to the panel launch is that prefix
// length, `max_d` the d of job 0. The in-block update launches take the runs
// of equal d ("classes") by value, so that their grids cover exactly the
// blocks that exist: a grid sized for the largest job times the job count
// would dispatch mostly empty workgroups.
constexpr int kQrMaxClasses = 16;
struct QrClasses {
    int32_t n;
    int32_t d[kQrMaxClasses];
    int32_t first[kQrMaxClasses];   // index of the class's first job
    int32_t count[kQrMaxClasses];
};
enum QrGridKind { QG_DOTS = 0, QG_REDUCE = 1, QG_UPDATE = 2, QG_TALL = 3 };

// Rows per workgroup of the tall-panel path (qr_tall_*): a panel's rows are
// split over ceil(L / kQrTallRows) workgroups.
constexpr int kQrTallRows = 256;

hipError_t launch_qr_panel(const QrJob* jobs, int njobs, int p, int max_d, hipStream_t s);
// The same panel factorisation with the rows of each panel spread over
// workgroups of kQrTallRows rows, all resident at once (one cooperative
// launch, a grid-wide barrier per column): for few, tall panels. C holds the
// runs of equal order of the first njobs jobs. qr_tall_blocks gives the
// workgroups it needs (-1 if C needs more than one launch) and
// qr_coop_capacity how many the device holds; launch_qr_panel_tall returns
// hipErrorInvalidValue without launching anything when they do not fit.
int qr_tall_blocks(const std::vector<QrClasses>& C, int p);
int qr_coop_capacity();
hipError_t launch_qr_panel_tall(const QrJob* jobs, int njobs, const std::vector<QrClasses>& C, int p, int max_d,
                                hipStream_t s);
hipError_t launch_qr_dots(const QrJob* jobs, const QrClasses& C, int p, hipStream_t s);
hipError_t launch_qr_reduce(const QrJob* jobs, const QrClasses& C, int p, hipStream_t s);
hipError_t launch_qr_update(const QrJob* jobs, const QrClasses& C, int p, hipStream_t s);
hipError_t launch_qr_init_q(const QrJob* jobs, int njobs, int max_d, hipStream_t s);
// Yb of outer block b for the first njobs jobs (those with d > b NB).
hipError_t launch_qr_copy_block(const QrJob* jobs, int njobs, int b, int max_d, hipStream_t s);

// -------------------------------------------------------------- health ----

// One matrix of the state checks: W, M and v scanned in chunks of kEwChunk.
struct HealthSeg {
    const float* W;
    const void* M;
    const float* v;
    int64_t n;            // elements
    int64_t chunk_begin;  // first chunk of this matrix in the launch
    int32_t m_bf16;
    int32_t out;          // index of the matrix's record (input order)
};
// Per-chunk partial statistics of v and non-finite count of W, M, v.
struct HealthPartial {
    double sabs, s, s2;
    float vmin, vmax;
    int64_t nonfinite;
};
// Per-matrix record: sums in float64, extremes, and the orthogonality drifts
// of U and V as float bit patterns (non-negative, so integer order is float
// order and the maximum can be taken with an integer atomic).
struct HealthOut {
    double sabs, s, s2;
    float vmin, vmax;
    uint32_t drift_u, drift_v;
    int64_t nonfinite;
    int64_t n;
};
// max |G - I| of one d x d Gram matrix G = X^T X into out[out].drift_u or _v.
struct DriftJob {
    const float* G;
    int32_t d;
    int32_t out;
    int32_t which;   // 0: U, 1: V
};
// X <- 1.5 X - 0.5 P over n contiguous elements (a Newton-Schulz step on a
// block of rows, P = X G for those rows).
struct NsJob {
    float* X;
    const float* P;
    int64_t n;
};

hipError_t launch_health_clear(HealthOut* out, int n, hipStream_t s);
hipError_t launch_health_partials(const HealthSeg* segs, int nseg, int64_t chunks, HealthPartial* part,
                                  hipStream_t s);
hipError_t launch_health_final(const HealthSeg* segs, int nseg, const HealthPartial* part, HealthOut* out,
                               hipStream_t s);
hipError_t launch_drift(const DriftJob* jobs, int njobs, int max_d, HealthOut* out, hipStream_t s);
hipError_t launch_ns_combine(const NsJob* jobs, int njobs, int64_t max_n, hipStream_t s);

// Strided copy of columns [c0, d) of X into Z (both d x d, row stride d):
// the completion block of the refresh input.
struct CopyJob {
    const float* src;
    float* dst;
    int32_t d;
    int32_t c0;
};
hipError_t launch_copy_cols(const CopyJob* jobs, int njobs, int max_d, hipStream_t s);

// Splits used by the in-block reflector-transpose product over `rows` rows.
__host__ __device__ inline int qr_splits(int rows) {
    int s = (rows + 255) / 256;
    return s < kQrMaxSplits ? (s < 1 ? 1 : s) : kQrMaxSplits;
}
__host__ __device__ inline int qr_chunk(int rows, int splits) {
    int c = (rows + splits - 1) / splits;
    return (c + 1) & ~1;
}

// Columns of Z that panel p of a d x d factorisation updates directly: the
// rest of its outer block (the columns past the block are updated once per
// block).
__host__ __device__ inline int qr_inblock_cols(int d, int p) {
    const int k = p * kQrPB;
    if (k >= d) return 0;
    const int jb = d - k < kQrPB ? d - k : kQrPB;
    const int end_blk = (p / kQrPanelsPerBlock + 1) * kQrNB;
    const int end = end_blk < d ? end_blk : d;
    return end - k - jb;
}

// Blocks one job contributes to a per-panel launch: reflector-transpose
// products (512 columns x one row split per block), their reduction (64
// columns per block) and the in-block update (128 x 128 tiles).
__host__ __device__ inline int qr_blocks_per_job(int kind, int d, int p) {
    if (kind == QG_TALL) {
        const int L = d - p * kQrPB;
        return L > 0 ? (L + kQrTallRows - 1) / kQrTallRows : 0;
    }
    const int ncols = qr_inblock_cols(d, p);
    if (ncols <= 0) return 0;
    const int L = d - p * kQrPB;
    if (kind == QG_DOTS) return ((ncols + 511) / 512) * qr_splits(L);
    if (kind == QG_REDUCE) return (ncols + kQrReduceCols - 1) / kQrReduceCols;
    return ((L + kQrTile - 1) / kQrTile) * ((ncols + kQrTile - 1) / kQrTile);
}

__host__ __device__ inline int qr_total_blocks(const QrClasses& C, int kind, int p) {
    int t = 0;
    for (int c = 0; c < C.n; ++c) t += qr_blocks_per_job(kind, C.d[c], p) * C.count[c];
    return t;
}

// Block id -> (job, block within the job); false for no such block.
__host__ __device__ inline bool qr_locate(const QrClasses& C, int kind, int p, int bid, int& job, int& local) {
    for (int c = 0; c < C.n; ++c) {
        const int per = qr_blocks_per_job(kind, C.d[c], p);
        const int tot = per * C.count[c];
        if (bid < tot) {
            job = C.first[c] + bid / per;
            local = bid % per;
            return true;
        }
        bid -= tot;
    }
    return false;
}

}  // namespace matopt
