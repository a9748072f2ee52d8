/*
 * matopt.h -- C ABI of the MI355X (gfx950) rotated-basis matrix-optimizer step.
 *
 * What the library computes, per whole weight matrix W (m x n) with gradient G
 * (sources cited by page title and section):
 *
 *   t <- t + 1
 *   M <- beta1 M + (1 - beta1) G                    momentum matrix, original space
 *        ("Pipeline parallelism and gradient staleness optimisation in
 *        distributed training", section 2.2: one momentum matrix per weight
 *        matrix; "Large-model distributed optimisation: three-layer decoupling
 *        of communication, memory and compute", section 2.2: EMA form)
 *   if K > 0 and (t - 1) mod K == 0:  refresh U, V  (pipeline-staleness page,
 *        section 2.2 power iteration + QR, section 4.2 period K)
 *   G~ = U^T G V,  m~ = U^T M V                     two-sided rotation (section 2.2)
 *   v  <- beta2 v + (1 - beta2) G~^2                three-layer page, section 2.1;
 *                                                   G~ squared in fp32 (section 5.2)
 *   u  =  m~ / (sqrt(v) + eps)                      pipeline-staleness page, 2.1
 *   W  <- W - lr U u V^T
 *
 * Refresh (orthogonal iteration with positive-diagonal QR), r = min(m, n):
 *   for (X, A) in ((U, M M^T), (V, M^T M)), power_iters times:
 *       Y = A X[:, :r]  (formed as M (M^T X_r) or M^T (M X_r))
 *       Z = [Y | X[:, r:]]                          previous-basis completion
 *       X = Q of Z = QR with diag(R) > 0 (a zero diagonal counts as positive)
 *
 * Matrices are packed into micro-groups in longest-processing-time order of
 * the cost m*n*(m+n), each group's fp32 gradient payload sum(4 m n) capped by
 * capacity_bytes (Canzona page, section 3.2.2 micro-group scheduling, section
 * 6.1: 512 MB-class groups). One step runs the groups one after another on the
 * caller's stream, each phase of a group as one grouped launch. A refresh is
 * batched separately, over as many matrices as refresh_capacity_bytes of QR
 * scratch allows, since its latency-bound QR panels need many matrices in
 * flight to fill the GPU.
 *
 * Conventions for every call:
 *  - All matrices are dense row-major with row stride equal to their column
 *    count (W, G, M, v: stride n; U: stride m; V: stride n).
 *  - Device pointers are HIP device (or managed) memory of the current device;
 *    host pointers are ordinary host memory. The library allocates no device
 *    memory: every tensor and the workspace belong to the caller and must
 *    outlive the group.
 *  - `stream` is a hipStream_t passed as void*; NULL means the default stream.
 *    step/refresh only enqueue work (no host synchronisation, no allocation).
 *  - A group is not thread-safe. Distinct groups are independent. Pointers of
 *    different matrices (and the workspace) must not overlap.
 *  - Errors: a negative opt_status is returned synchronously for argument or
 *    state errors; opt_last_error() gives a text (thread-local, valid until the
 *    next call on this thread). Asynchronous device faults surface as OPT_EHIP
 *    on a later call. NaN/Inf in inputs propagate (no masking).
 */
#ifndef MATOPT_H_
#define MATOPT_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct opt_group_s* opt_group_t;

typedef enum {
    OPT_OK = 0,
    OPT_EINVAL = -1,        /* bad argument: null/misshaped/aliased pointer, bad hyper-parameter */
    OPT_ENOWS = -2,         /* workspace smaller than opt_group_workspace_size() */
    OPT_EHIP = -3,          /* a HIP runtime call failed (text carries hipGetErrorString) */
    OPT_EUNSUPPORTED = -4,  /* dtype or size outside what the kernels implement */
    OPT_ESTATE = -5         /* call on a group in an unusable state */
} opt_status;

typedef enum { OPT_F32 = 0, OPT_BF16 = 1 } opt_dtype;

/* One whole matrix (the atomicity constraint of the Canzona page, section 2.1:
 * a matrix optimizer needs the entire matrix, never a shard). */
typedef struct {
    int64_t m, n;          /* rows, columns; 1 <= m, n <= OPT_MAX_DIM */
    float* W;              /* m x n fp32 master weights, updated in place */
    const float* G;        /* m x n fp32 gradient, read by every step (caller refills it) */
    void* M;               /* m x n momentum, fp32 or bf16 (M_dtype), updated in place; start at 0 */
    int32_t M_dtype;       /* opt_dtype */
    float* v;              /* m x n fp32 second moment in rotated coordinates; start at 0
                              (NULL allowed with OPT_FLAG_MUON, as for U and V) */
    float* U;              /* m x m fp32 orthonormal left basis, updated by refreshes; start at I
                              (bf16, 16-byte aligned, with OPT_FLAG_BF16_BASES: cast the pointer) */
    float* V;              /* n x n fp32 orthonormal right basis, likewise */
    float* Mt;             /* m x n fp32 momentum in rotated coordinates, used only with
                              OPT_FLAG_ROTATED_MOMENTUM (else must be NULL); its content is
                              rebuilt by the first step, so it needs no initial value */
} opt_matrix_desc;

/* opt_hparams.flags */
enum {
    /* Carry the rotated momentum m~ = U^T M V across steps of one basis epoch
     * instead of recomputing it: within an epoch U and V are fixed and M is an
     * EMA, so U^T M_t V = b1 m~_{t-1} + (1 - b1) U^T G_t V (the momentum matrix
     * and two-sided rotation of the Pipeline-parallelism page, section 2.2, with
     * the EMA of the three-layer decoupling page, section 2.2). A step then
     * needs two two-sided products instead of three. m~ is recomputed as
     * U^T M V on the first step, at every refresh, and after refresh_basis,
     * reorthonormalize or set_step; M is still kept in the original space for
     * the refreshes. Equal
     * to the method in exact arithmetic; m~ is stored in fp32 (with a bf16 M
     * it is therefore not rounded to bf16 between steps). */
    OPT_FLAG_ROTATED_MOMENTUM = 1u,
    /* Run the rotations on bfloat16 operands with fp32 accumulation (the
     * rotation matrices kept in 16-bit floats, as in the Pipeline-parallelism
     * page, section 3.1; bfloat16 rather than float16 so that one operand
     * format serves the bases, the bf16 momentum and the gradient). U, V stay
     * fp32 and are what the refresh updates; bf16 copies of U, U^T, V, V^T
     * live in the workspace and are rebuilt on the first step after a
     * refresh, a create, refresh_basis, reorthonormalize or set_step (a caller
     * that writes U or V itself must call opt_group_set_step afterwards). The
     * bf16 roundings: G, M, the bases, the right rotations X V, u and the
     * rotation back u V^T; G~, m~, v and W stay fp32. The first step of a
     * group (t = 1, where v = 0) uses the fp32 rotations: there u divides by
     * sqrt(v) + eps and bf16 roundoff in directions where G~ vanishes would
     * become full-size entries of u. With OPT_FLAG_ROTATED_MOMENTUM as well,
     * m~ is carried in Mt (fp32) as that flag describes and only G is rotated
     * on the steps that carry it. The workspace grows by the
     * bf16 bases, 4 (m m8 + n n8) bytes per matrix (m8, n8: m, n rounded up
     * to a multiple of 8). */
    OPT_FLAG_BF16_ROTATION = 2u,
    /* A second matrix optimizer on the same groups: the orthogonalised
     * momentum step (Muon-style; the Canzona page, sections 1 and 7, names
     * Muon and its orthogonalisation without a formula). M is the same EMA,
     * then O = the orthogonal polar factor of M approximated by ns_iters
     * steps of the cubic Newton-Schulz iteration X <- 1.5 X - 0.5 X X^T X
     * from X = M / ||M||_F (on the side with the smaller Gram matrix), and
     * W <- W - lr O. v, U, V are unused (may be NULL), as are beta2, eps, K
     * and power_iters; refresh_basis, health and reorthonormalize return
     * OPT_EUNSUPPORTED. Combines with OPT_FLAG_FP32_MFMA only. */
    OPT_FLAG_MUON = 4u,
    /* By default the fp32 products of the rotations and of the refresh run on
     * bf16 MFMAs (2.5 PFLOP/s dense against 157 TFLOP/s for fp32), at fp32
     * accuracy:
     *  - every fp32 operand value splits exactly into three bf16 pieces
     *    hi = rb(x), mid = rb(x - hi), lo = x - hi - mid in registers, and the
     *    six piece products that matter (hi hi, hi mid, mid hi, hi lo, mid mid,
     *    lo hi) accumulate in fp32; the three left out are below 2^-23 of the
     *    product, about one fp32 rounding (the bf16x6 scheme of Henry, Tang
     *    and Heinecke, ARITH 2019);
     *  - a bf16 momentum (m and n multiples of 8, M 16-byte aligned, no
     *    other flag) is exactly bf16, so the product of M's chain with the
     *    larger flop count (U^T M when m > n, M V otherwise) needs only three
     *    products, against stored pieces of U^T or V^T (6 d^2 bytes per
     *    matrix, d = m or n, made with the U^T copy), in one fp32 chain.
     * The Newton-Schulz products of OPT_FLAG_MUON run the same way. This flag
     * keeps every one of these products on fp32 MFMAs. */
    OPT_FLAG_FP32_MFMA = 8u,
    /* With OPT_FLAG_BF16_ROTATION: U and V are stored in bfloat16 and are the
     * only copies of the bases (the Pipeline-parallelism page, section 3.1,
     * keeps the rotation matrices in 16 bits, about 15 % of the memory). The
     * descriptor's U and V point to bf16 m x m and n x n matrices, 16-byte
     * aligned, initialised to I. A refresh widens them into fp32 copies in
     * its scratch, runs the orthogonal iteration there and stores the result
     * rounded to nearest even. Every step rotates with the stored bases,
     * the first one included (there is no fp32 copy for it). Where m (n) is a
     * multiple of 8 the caller's U (V) also serves as the rotations' bf16
     * copy, so the workspace holds only U^T and V^T in bf16. Health checks
     * and re-orthonormalisation return OPT_EUNSUPPORTED. */
    OPT_FLAG_BF16_BASES = 16u
};

typedef struct {
    float beta1;              /* momentum EMA weight, 0 <= beta1 < 1 */
    float beta2;              /* second-moment EMA weight, 0 <= beta2 < 1 */
    float eps;                /* > 0 */
    float lr;                 /* finite */
    int32_t K;                /* refresh period in steps; 0 = no automatic refresh */
    int32_t power_iters;      /* orthogonal-iteration passes per refresh, >= 1 */
    uint64_t capacity_bytes;  /* micro-group cap on sum(4 m n); 0 selects 1 << 29 (512 MiB) */
    uint64_t refresh_capacity_bytes; /* cap on the refresh scratch of one refresh batch (the
                                        d x d QR inputs and their scratch); 0 selects the
                                        largest of 4 GiB, the bytes of the copies of the bases
                                        and the step scratch (which the refresh buffers
                                        overlay) and the bytes of the group's tensors (W, G, M,
                                        v, U, V, Mt). A matrix larger than the cap forms a
                                        batch alone. */
    uint32_t flags;           /* OPT_FLAG_* bits; others must be 0 */
    int32_t ns_iters;         /* Newton-Schulz iterations of OPT_FLAG_MUON, >= 1 there; else ignored */
} opt_hparams;

#define OPT_MAX_DIM 16384       /* largest m or n the QR panel kernel supports */
#define OPT_MAX_MATRICES 65536

/* Bytes of device workspace a group over these matrices needs (host only).
 * The workspace holds the device-side work lists, then either the copies of
 * the bases followed by the scratch of one micro-group (reused by every group
 * in turn), or, during a refresh (and the drift check of opt_group_health),
 * the buffers of one refresh batch, which overlay both: the total is the
 * tables plus the larger of the two. The copies:
 * with fp32 rotations (no flag, or OPT_FLAG_ROTATED_MOMENTUM alone) U^T in
 * fp32, 4 m^2 bytes per matrix, so that U^T G and U^T M read rows of U^T,
 * and without flags, for a bf16 M with both sides multiples of 8, the three
 * bf16 pieces of U^T (m > n) or V^T (else), 6 d^2 bytes (none with
 * OPT_FLAG_FP32_MFMA);
 * with OPT_FLAG_BF16_ROTATION the bf16 bases described there. They are
 * rebuilt on the first step after a create, a refresh, refresh_basis,
 * reorthonormalize, health or set_step: a caller that writes U or V itself
 * must call opt_group_set_step afterwards. */
opt_status opt_group_workspace_size(const opt_matrix_desc* descs, int32_t count,
                                    const opt_hparams* hp, uint64_t* bytes);

/* The parts of that workspace (host only), in bytes: parts[0] the work
 * lists, parts[1] the copies of the bases, parts[2] the step scratch,
 * parts[3] the largest refresh batch's buffers. The workspace size is
 * parts[0] + max(parts[1] + parts[2], parts[3]). `parts` has 4 entries. */
opt_status opt_group_workspace_parts(const opt_matrix_desc* descs, int32_t count,
                                     const opt_hparams* hp, uint64_t* parts);

/* Validate, plan the micro-groups, lay out the workspace and upload the work
 * lists with an asynchronous copy on `stream`. `workspace` must be device
 * memory of at least opt_group_workspace_size() bytes, 256-byte aligned.
 * The step counter starts at t = 0. On success *out receives the group. */
opt_status opt_group_create(const opt_matrix_desc* descs, int32_t count, const opt_hparams* hp,
                            void* workspace, uint64_t workspace_bytes, void* stream,
                            opt_group_t* out);

/* One optimizer step over every matrix (see the top of this file). Enqueues
 * on `stream`; t is incremented on the host before enqueueing. */
opt_status opt_group_step(opt_group_t g, void* stream);

/* Refresh U and V of every matrix from the current M with `power_iters`
 * passes (>= 1); W, M, v and t are untouched. Enqueues on `stream`. */
opt_status opt_group_refresh_basis(opt_group_t g, int32_t power_iters, void* stream);

/* ---- state checks and basis repair ---------------------------------------
 * Both use the group's workspace like step and refresh: calls on one group
 * must not overlap in time (use one stream, or synchronise between them). */

/* Health of one matrix. The Pipeline-parallelism page (section 5.1) checks
 * that the rotation matrices stay orthogonal; the three-layer decoupling page
 * flags a contaminated second moment when std(v) / mean(|v|) exceeds 10
 * (section 4.3) and watches min(v) (section 4.4). */
typedef struct {
    double orth_U;      /* max_ij |(U^T U - I)_ij|, from an fp32 Gram matrix (floor ~1e-6); inf if not finite */
    double orth_V;      /* the same for V */
    double v_mean_abs;  /* mean |v| */
    double v_std;       /* population standard deviation of v */
    double v_min;       /* minimum of v (NaN entries skipped; they are counted below) */
    double v_max;
    int64_t nonfinite;  /* NaN and +-Inf entries of W, M and v */
} opt_health;

/* Fills out[i] for every matrix i (input order, `count` entries as given at
 * create). Enqueues on `stream`, then synchronises it. Sums are float64. */
opt_status opt_group_health(opt_group_t g, opt_health* out, void* stream);

/* Restores the orthonormality of every U and V with `iters` (>= 0)
 * Newton-Schulz steps X <- X (3 I - X^T X) / 2, which converge quadratically
 * to the polar factor X (X^T X)^(-1/2) (the Pipeline-parallelism page,
 * section 5.1) when ||X^T X - I||_2 < 1 (check with opt_group_health first:
 * orth < 1 / (order) suffices); one step takes a drift e to about 1.5 e^2,
 * down to the fp32 floor. Enqueues on `stream`. */
opt_status opt_group_reorthonormalize(opt_group_t g, int32_t iters, void* stream);

/* Step counter, for checkpoint/resume (all other state is caller-owned;
 * set_step also marks the workspace copies of U and V for a rebuild). */
opt_status opt_group_get_step(opt_group_t g, int64_t* t);
opt_status opt_group_set_step(opt_group_t g, int64_t t);   /* t >= 0 */
opt_status opt_group_set_lr(opt_group_t g, float lr);      /* finite */

/* Micro-group plan, host only (pointers in descs are not read). order[k] is
 * the input index of the k-th matrix in LPT order; group_of[i] the micro-group
 * of input matrix i; *num_groups the number of groups. Arrays have `count`
 * entries; any output pointer may be NULL. */
opt_status opt_plan(const opt_matrix_desc* descs, int32_t count, const opt_hparams* hp,
                    int32_t* order, int32_t* group_of, int32_t* num_groups);

/* Per-phase timing with HIP events recorded on the step's stream around every
 * launch of the phase. Phases: */
enum {
    OPT_PHASE_MOMENTUM = 0,   /* momentum EMA (elementwise) */
    OPT_PHASE_REFRESH = 1,    /* whole basis refresh (products + QR) */
    OPT_PHASE_ROT_LEFT = 2,   /* U^T G, U^T M                 (grouped GEMM) */
    OPT_PHASE_ROT_RIGHT = 3,  /* (U^T G) V, (U^T M) V         (grouped GEMM) */
    OPT_PHASE_ADAM = 4,       /* v and u in the rotated basis (elementwise) */
    OPT_PHASE_BACK_LEFT = 5,  /* U u                          (grouped GEMM) */
    OPT_PHASE_BACK_RIGHT = 6, /* W -= lr (U u) V^T            (grouped GEMM + apply) */
    OPT_PHASE_ORTHO = 7,      /* OPT_FLAG_MUON: norm, Newton-Schulz products and combines, apply */
    OPT_PHASE_ROT_PIECED = 8, /* bf16 M's pieced product (U^T M or M V) and the M^T it reads */
    OPT_NUM_PHASES = 9
};
/* enable != 0 starts recording and clears the totals; 0 stops. Enabling
 * creates the HIP events for 64 steps' worth of phase scopes up front (so a
 * step never creates one); a call on the group's device. */
opt_status opt_group_set_timing(opt_group_t g, int32_t enable);
/* Synchronises with the last recorded event, folds the records into the
 * totals and frees the event pool for the next 64 steps, then writes for
 * each phase the summed milliseconds and the number of kernels launched in
 * the timed scopes since timing was enabled (arrays of OPT_NUM_PHASES
 * entries; either may be NULL). Returns OPT_ESTATE (after writing the totals)
 * if more scopes were entered between two reads than the pool holds: the
 * totals then miss the scopes that found no event. Every scope counts its grouped GEMM and elementwise launches; the
 * refresh scope counts its grouped GEMMs (Gram products and the QR's outer-
 * block updates), not the QR's panel and in-block kernels. */
opt_status opt_group_read_timing(opt_group_t g, double* ms, int64_t* launches);
/* The same totals per micro-group: ms[k] is the summed milliseconds of every
 * timed scope of micro-group k (its momentum, rotation, Adam and update
 * phases, and its pieced product), in the plan's group order (opt_plan's
 * group_of); count must equal the number of micro-groups. The refresh and
 * the copies of the bases run over refresh batches, not micro-groups, and
 * are not included. Folds the records like opt_group_read_timing (either
 * call reads what the other has not), with the same overflow report. The
 * Canzona page (section 6.1) sizes micro-groups for throughput, which this
 * reads off per group. */
opt_status opt_group_read_group_timing(opt_group_t g, double* ms, int32_t count);

void opt_group_destroy(opt_group_t g);   /* NULL is ignored; does not synchronise */

const char* opt_last_error(void);

/* ---- building blocks, exported for testing and reuse ------------------- */

/* C = alpha * op(A) op(B) + beta * C on device memory, fp32 accumulate.
 * op(A) is M x K: A is stored row-major as M x K (trans_a = 0, row stride
 * lda >= K) or as K x M (trans_a = 1, lda >= M). op(B) is K x N: B stored as
 * K x N (trans_b = 0, ldb >= N) or N x K (trans_b = 1, ldb >= K). A and B
 * are fp32 or bf16 (a_dtype, b_dtype); C is fp32 (ldc >= N). beta == 0 does
 * not read C. M, N, K >= 0 (an empty product only scales C). */
opt_status opt_gemm(int32_t trans_a, int32_t trans_b, int64_t M, int64_t N, int64_t K,
                    float alpha, const void* A, int32_t a_dtype, int64_t lda,
                    const void* B, int32_t b_dtype, int64_t ldb,
                    float beta, float* C, int64_t ldc, void* stream);

/* opt_gemm on bf16 MFMAs at fp32 accuracy (the bf16x6 scheme of Henry, Tang
 * and Heinecke, ARITH 2019, as the step uses it by default): each fp32
 * operand value splits exactly into three bf16 pieces, the six piece products
 * that matter accumulate in fp32, and the ones left out are below 2^-23 of
 * each product. Same arguments as opt_gemm; the supported layouts are
 * (trans_a, trans_b, a_dtype, b_dtype) = (0, 0, F32, F32), (1, 0, F32, F32),
 * (0, 1, F32, F32), (0, 0, F32, BF16), (0, 0, BF16, F32) and
 * (1, 0, BF16, F32); with a bf16
 * operand, which is its own high piece, three piece products. Others return
 * OPT_EUNSUPPORTED. */
opt_status opt_gemm_x6(int32_t trans_a, int32_t trans_b, int64_t M, int64_t N, int64_t K,
                       float alpha, const void* A, int32_t a_dtype, int64_t lda,
                       const void* B, int32_t b_dtype, int64_t ldb,
                       float beta, float* C, int64_t ldc, void* stream);

/* C = alpha * A B^T + beta * C with bfloat16 operands and fp32 accumulation
 * (the product of the bf16-rotation variant, section 3.1 of the pipeline-
 * parallelism page keeping the rotation matrices in 16-bit floats). A is M x K
 * and B is N x K, both bf16, row-major with k contiguous (row strides lda,
 * ldb >= K); K, lda and ldb must be multiples of 8 and A, B 16-byte aligned
 * (OPT_EINVAL otherwise). C is M x N row-major (ldc >= N): fp32 when c_dtype
 * is OPT_F32, or bf16 rounded to nearest even when c_dtype is OPT_BF16, which
 * requires beta == 0. beta == 0 does not read C. M, N, K >= 0; an empty
 * product only scales C. Enqueued on `stream`; no allocation. */
opt_status opt_gemm_bf16(int64_t M, int64_t N, int64_t K, float alpha, const void* A, int64_t lda,
                         const void* B, int64_t ldb, float beta, void* C, int32_t c_dtype, int64_t ldc,
                         void* stream);

/* Q = the positive-diagonal-R orthonormal factor of the d x d fp32 matrix Z
 * (row-major, stride d). Z is overwritten with the Householder factorisation
 * (R on and above the diagonal, reflectors below). Q must not overlap Z. The
 * block products run on bf16 MFMAs at fp32 accuracy, as in the refresh.
 * `workspace` is device memory of opt_orthonormalize_workspace_size(d) bytes. */
opt_status opt_orthonormalize_workspace_size(int64_t d, uint64_t* bytes);
opt_status opt_orthonormalize(float* Z, float* Q, int64_t d, void* workspace,
                              uint64_t workspace_bytes, void* stream);

/* opt_orthonormalize without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc). The QR job record and scratch live in a
 * fixed device array inside the library, sized for one matrix of order
 * OPT_STATIC_MAX_DIM (about 22 MiB); every GPU the library runs on holds its
 * own copy until the process ends. Same kernels and results as
 * opt_orthonormalize. d > OPT_STATIC_MAX_DIM returns OPT_EUNSUPPORTED; no
 * device memory is allocated or freed. The array keeps whatever the last call
 * left in it (no kernel relies on its contents at entry), and all calls on one
 * GPU share it: calls that overlap in time on one GPU (different streams or
 * host threads without synchronisation between them) race and must not be
 * made. Enqueues on `stream`. */
#define OPT_STATIC_MAX_DIM 4096
opt_status opt_orthonormalize_static(float* Z, float* Q, int64_t d, void* stream);

/* ---- cross-rank planners (host only; no device memory, no stream) -------
 * A job that shards its matrices over several ranks plans once, on the host,
 * which rank steps which whole matrix; each rank then runs a group over its
 * share. Costs are the caller's (e.g. flops per step: 6 m n (m + n) for the
 * rotations plus the amortised refresh). Every floating-point sum is taken
 * left to right in the order described, so the integer results are
 * reproducible across implementations. */

/* Alpha-balanced greedy LPT partition of data-parallel buckets over `ranks`
 * ranks (the Canzona page, section 3.2.1, with the geometric alignment of
 * section 4.2). Parameter i has cost cost[i] >= 0 (finite); bucket b holds the
 * consecutive parameters bucket_begin[b] .. bucket_begin[b+1]-1
 * (bucket_begin has nbuckets + 1 non-decreasing entries, from 0 to nparams).
 * Buckets are placed by decreasing total cost W_b (ties in input order). For
 * each bucket, with L_r the rank loads so far and T = sum_r L_r / ranks the
 * mean of those loads (the section's deficit against the ideal mean), the
 * target share of rank r is
 * (1 - alpha) / ranks + alpha * max(0, T - L_r) / sum_s max(0, T - L_s)
 * (1 / ranks when that sum is 0, e.g. for the first bucket). The bucket is cut into `ranks` consecutive
 * ranges, rank 0 first, only at parameter boundaries: boundary r (1 <= r <
 * ranks) is the prefix of the bucket whose cost is nearest to W_b times the
 * summed shares of ranks < r, searched from the previous boundary on, ties to
 * the shorter prefix. Ranges may be empty. Outputs: owner[i] (nparams
 * entries) and, if not NULL, load[r] (ranks entries), the summed cost of
 * each rank's parameters. 0 <= alpha <= 1; ranks >= 1. */
opt_status opt_partition_dp(const double* cost, int64_t nparams, const int64_t* bucket_begin,
                            int32_t nbuckets, int32_t ranks, double alpha, int32_t* owner,
                            double* load);

/* Micro-groups with host ranks for tensor-parallel matrices (the Canzona
 * page, section 3.2.2): parameters sorted by decreasing cost (ties in input
 * order) are added in turn to the current micro-group; when the group's
 * summed bytes would exceed `capacity_bytes` (0 selects 512 MiB) a new group
 * is opened first (a parameter larger than the capacity forms a group alone).
 * Inside a group each parameter goes to the host rank with the least cost
 * assigned in that group so far (a min-heap over the ranks; ties to the
 * lowest rank). Outputs (n entries each, any may be NULL): order[k], the
 * input index of the k-th parameter in that order; group_of[i]; host_of[i];
 * *num_groups. ranks >= 1; cost[i] >= 0 finite. */
opt_status opt_plan_host_ranks(const double* cost, const uint64_t* bytes, int64_t n, int32_t ranks,
                               uint64_t capacity_bytes, int32_t* order, int32_t* group_of,
                               int32_t* host_of, int32_t* num_groups);

#ifdef __cplusplus
}
#endif
#endif /* MATOPT_H_ */
