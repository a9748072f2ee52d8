// Blocked Householder QR with explicit Q for the basis refresh (gfx950).
//
// The refresh needs the orthonormal factor Q of Z = QR with diag(R) > 0 for
// d x d inputs up to d = 12288 that are often numerically rank deficient in
// fp32 (products of the Gram matrix with the previous basis). Householder
// reflections keep Q orthonormal to working precision regardless of the
// conditioning of Z, which Cholesky- or Gram-Schmidt-based schemes do not.
//
// Factorisation, panel by panel (width PB = 32), right-looking:
//   1. qr_panel   one 512-thread workgroup per matrix factorises the L x PB
//                 panel column by column (two passes over the panel rows per
//                 column, two block reductions), stores the reflectors below
//                 the diagonal of Z, R on and above it, and builds the
//                 upper-triangular T of the compact WY form
//                 H_0 ... H_{jb-1} = I - Y T Y^T by the forward recurrence
//                 T[:j, j] = -tau_j T[:j, :j] (Y[:, :j]^T v_j).
//   2. qr_dots    W = Y^T C for the trailing block C, split over rows into
//                 partial sums (fp32 MFMA 32x32x2 straight from global memory:
//                 both operands are read along their contiguous dimension).
//   3. qr_reduce  sums the partials and applies T^T: W2 = T^T W.
//   4. qr_update  C -= Y W2 on the grouped GEMM tile (unit-lower A loader).
// Q formation (backward accumulation): X = diag(sign(R_ii)) (qr_init_q, so
// the sign convention costs nothing), then for panels from last to first
// X[k:, k:] -= Y T (Y^T X[k:, k:]) with the same three kernels (q_mode 1).
//
// Several matrices are factorised in lock step: every launch covers all
// matrices that still have panel p, which are a prefix of the job array
// sorted by d descending.
#include "internal.h"

namespace matopt {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

namespace {

constexpr int PB = kQrPB;
constexpr int PT = kQrPanelThreads;
constexpr int NW = PT / 64;

struct PanelShared {
    float red[NW][PB];
    float w[PB];
    float T[PB][PB + 1];
    float rsig[NW];
    float alpha;
};

struct PanelCtx {
    float* A;      // top-left of the panel (row k, column k of Z)
    int64_t ld;
    int L;         // rows of the panel
    int jb;        // columns of the panel
    bool vec;      // full-width panel with 16-byte aligned rows
};

__device__ __forceinline__ void load_row(const PanelCtx& c, int i, float (&a)[PB]) {
    const float* p = c.A + (int64_t)i * c.ld;
    if (c.vec) {
#pragma unroll
        for (int q = 0; q < PB / 4; ++q) {
            const f32x4 t = *(const f32x4*)(p + 4 * q);
            a[4 * q + 0] = t[0];
            a[4 * q + 1] = t[1];
            a[4 * q + 2] = t[2];
            a[4 * q + 3] = t[3];
        }
    } else {
#pragma unroll
        for (int q = 0; q < PB; ++q) a[q] = q < c.jb ? p[q] : 0.f;
    }
}

__device__ __forceinline__ void store_row(const PanelCtx& c, int i, const float (&a)[PB]) {
    float* p = c.A + (int64_t)i * c.ld;
    if (c.vec) {
#pragma unroll
        for (int q = 0; q < PB / 4; ++q) {
            f32x4 t;
            t[0] = a[4 * q + 0];
            t[1] = a[4 * q + 1];
            t[2] = a[4 * q + 2];
            t[3] = a[4 * q + 3];
            *(f32x4*)(p + 4 * q) = t;
        }
    } else {
#pragma unroll
        for (int q = 0; q < PB; ++q)
            if (q < c.jb) p[q] = a[q];
    }
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

// Sum 32 per-thread values over the workgroup into sh.w[0..31].
// Within a wavefront this is a reduce-scatter: at each of five exchange steps
// a lane keeps one half of its remaining values (the upper half when its
// partner bit is set) and adds the partner's copy of that half, so after
// 16+8+4+2+1 shuffles lane l holds the sum over its 32 partner lanes of
// value (l >> 1) & 31; one more exchange with lane l^1 completes the sum.
__device__ __forceinline__ void block_sum32(float (&v)[PB], PanelShared& sh) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    float r16[16];
    {
        const bool hi = lane & 32;
#pragma unroll
        for (int c = 0; c < 16; ++c) {
            const float keep = hi ? v[16 + c] : v[c];
            const float give = hi ? v[c] : v[16 + c];
            r16[c] = keep + __shfl_xor(give, 32, 64);
        }
    }
    float r8[8];
    {
        const bool hi = lane & 16;
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const float keep = hi ? r16[8 + c] : r16[c];
            const float give = hi ? r16[c] : r16[8 + c];
            r8[c] = keep + __shfl_xor(give, 16, 64);
        }
    }
    float r4[4];
    {
        const bool hi = lane & 8;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const float keep = hi ? r8[4 + c] : r8[c];
            const float give = hi ? r8[c] : r8[4 + c];
            r4[c] = keep + __shfl_xor(give, 8, 64);
        }
    }
    float r2[2];
    {
        const bool hi = lane & 4;
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const float keep = hi ? r4[2 + c] : r4[c];
            const float give = hi ? r4[c] : r4[2 + c];
            r2[c] = keep + __shfl_xor(give, 4, 64);
        }
    }
    float r1;
    {
        const bool hi = lane & 2;
        const float keep = hi ? r2[1] : r2[0];
        const float give = hi ? r2[0] : r2[1];
        r1 = keep + __shfl_xor(give, 2, 64);
    }
    r1 += __shfl_xor(r1, 1, 64);
    if ((lane & 1) == 0) sh.red[wave][(lane >> 1) & 31] = r1;
    __syncthreads();
    if (threadIdx.x < PB) {
        float s = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) s += sh.red[w][threadIdx.x];
        sh.w[threadIdx.x] = s;
    }
    __syncthreads();
}

// Column J of the panel (J is a compile-time constant so that every register
// array index below is static).
template <int J>
__device__ __forceinline__ void column_step(const PanelCtx& c, PanelShared& sh) {
    if (J >= c.jb) return;
    const int tid = threadIdx.x;

    float sig = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) sig += sh.rsig[w];
    const float alpha = sh.alpha;
    float beta, tau, scale;
    if (sig == 0.f) {
        beta = alpha;
        tau = 0.f;
        scale = 0.f;
    } else {
        const float nrm = __builtin_sqrtf(alpha * alpha + sig);
        beta = -__builtin_copysignf(nrm, alpha);
        tau = (beta - alpha) / beta;
        scale = 1.f / (alpha - beta);
    }

    // Pass 1: dots of v_J with every other panel column (trailing columns give
    // the update weights, leading columns hold earlier reflectors and give the
    // inner products needed for T).
    float part[PB];
#pragma unroll
    for (int q = 0; q < PB; ++q) part[q] = 0.f;
    for (int i = tid; i < c.L; i += PT) {
        if (i < J) continue;
        float a[PB];
        load_row(c, i, a);
        const float vi = (i == J) ? 1.f : a[J] * scale;
#pragma unroll
        for (int q = 0; q < PB; ++q)
            if (q != J) part[q] += vi * a[q];
    }
    block_sum32(part, sh);

    if (tid < J) {
        float s = 0.f;
        for (int l = tid; l < J; ++l) s += sh.T[tid][l] * sh.w[l];
        sh.T[tid][J] = -tau * s;
    } else if (tid == J) {
        sh.T[J][J] = tau;
    }

    float tw[PB];
#pragma unroll
    for (int q = 0; q < PB; ++q) tw[q] = q > J ? tau * sh.w[q] : 0.f;

    // Pass 2: apply H_J to the trailing columns, store v_J and beta, and
    // accumulate the squared norm of the next column below its diagonal.
    float sig_part = 0.f;
    for (int i = tid; i < c.L; i += PT) {
        if (i < J) continue;
        float a[PB];
        load_row(c, i, a);
        const float vi = (i == J) ? 1.f : a[J] * scale;
#pragma unroll
        for (int q = J + 1; q < PB; ++q) a[q] -= vi * tw[q];
        a[J] = (i == J) ? beta : vi;
        store_row(c, i, a);
        if (J + 1 < PB && J + 1 < c.jb) {
            if (i > J + 1) sig_part += a[J + 1] * a[J + 1];
            else if (i == J + 1) sh.alpha = a[J + 1];
        }
    }
    const float ws = wave_sum(sig_part);
    if ((tid & 63) == 0) sh.rsig[tid >> 6] = ws;
    __syncthreads();
}

template <int J>
struct Columns {
    __device__ __forceinline__ static void run(const PanelCtx& c, PanelShared& sh) {
        column_step<J>(c, sh);
        Columns<J + 1>::run(c, sh);
    }
};
template <>
struct Columns<PB> {
    __device__ __forceinline__ static void run(const PanelCtx&, PanelShared&) {}
};

__global__ __launch_bounds__(PT) void qr_panel_kernel(const QrJob* __restrict__ jobs, int p) {
    __shared__ PanelShared sh;
    const QrJob Jb = jobs[blockIdx.x];
    const int k = p * PB;
    if (k >= Jb.d) return;
    PanelCtx c;
    c.ld = Jb.d;
    c.A = Jb.Z + (int64_t)k * c.ld + k;
    c.L = Jb.d - k;
    c.jb = min(PB, Jb.d - k);
    c.vec = (c.jb == PB) && (Jb.d % 4 == 0);
    const int tid = threadIdx.x;

    for (int e = tid; e < PB * (PB + 1); e += PT) (&sh.T[0][0])[e] = 0.f;
    float sig_part = 0.f;
    for (int i = tid; i < c.L; i += PT) {
        const float x = c.A[(int64_t)i * c.ld];
        if (i > 0) sig_part += x * x;
        else sh.alpha = x;
    }
    const float ws = wave_sum(sig_part);
    if ((tid & 63) == 0) sh.rsig[tid >> 6] = ws;
    __syncthreads();

    Columns<0>::run(c, sh);

    float* Tout = Jb.T + (int64_t)p * PB * PB;
    for (int e = tid; e < PB * PB; e += PT) Tout[e] = sh.T[e / PB][e % PB];
}

// Partial products W_s = Y[rows of split s]^T C[rows of split s].
// A wavefront owns a 32 x 128 block of W (four 32x32 MFMA accumulators that
// share the Y operand); lane l supplies Y[row + l/32][l%32] and
// C[row + l/32][col + l%32], i.e. 128-byte row segments of both matrices.
__global__ __launch_bounds__(256) void qr_dots_kernel(const QrJob* __restrict__ jobs, int p,
                                                     int q_mode) {
    const QrJob Jb = jobs[blockIdx.z];
    const int k = p * PB;
    if (k >= Jb.d) return;
    const int d = Jb.d;
    const int jb = min(PB, d - k), L = d - k;
    const int ncols = q_mode ? L : L - jb;
    if (ncols <= 0) return;
    const int splits = qr_splits(L), kc = qr_chunk(L, splits);
    const int s = blockIdx.y;
    if (s >= splits) return;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, h = lane >> 5, l32 = lane & 31;
    const int j0 = blockIdx.x * 512 + wave * 128;
    if (j0 >= ncols) return;
    const int r0 = s * kc, r1 = min(L, r0 + kc);
    const float* Y = Jb.Z + (int64_t)k * d + k;
    const float* C = q_mode ? Jb.X + (int64_t)k * d + k : Jb.Z + (int64_t)k * d + k + jb;

    f32x16 acc[4];
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[b][r] = 0.f;

#pragma unroll 4
    for (int i = r0; i < r1; i += 2) {
        const int row = i + h;
        float y = 0.f;
        float x[4] = {0.f, 0.f, 0.f, 0.f};
        if (row < r1) {
            if (l32 < jb) y = row < l32 ? 0.f : (row == l32 ? 1.f : Y[(int64_t)row * d + l32]);
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const int col = j0 + 32 * b + l32;
                if (col < ncols) x[b] = C[(int64_t)row * d + col];
            }
        }
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[b] = __builtin_amdgcn_mfma_f32_32x32x2f32(y, x[b], acc[b], 0, 0, 0);
    }

    float* part = Jb.part + (int64_t)s * PB * d;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        const int j = j0 + 32 * b + l32;
        if (j >= ncols) continue;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int cc = 8 * (r >> 2) + 4 * h + (r & 3);
            part[(int64_t)cc * d + j] = acc[b][r];
        }
    }
}

// W2[:, j] = T^T (sum_s W_s[:, j])  (factorisation)   or   T (...)  (Q formation).
__global__ __launch_bounds__(256) void qr_reduce_kernel(const QrJob* __restrict__ jobs, int p,
                                                       int q_mode) {
    __shared__ float Ts[PB][PB + 1];
    const QrJob Jb = jobs[blockIdx.y];
    const int k = p * PB;
    if (k >= Jb.d) return;
    const int d = Jb.d;
    const int jb = min(PB, d - k), L = d - k;
    const int ncols = q_mode ? L : L - jb;
    if (ncols <= 0) return;
    const float* Tp = Jb.T + (int64_t)p * PB * PB;
    for (int e = threadIdx.x; e < PB * PB; e += 256) Ts[e / PB][e % PB] = Tp[e];
    __syncthreads();
    const int j = blockIdx.x * 256 + threadIdx.x;
    if (j >= ncols) return;
    const int splits = qr_splits(L);
    float w[PB];
#pragma unroll
    for (int c = 0; c < PB; ++c) w[c] = 0.f;
    for (int s = 0; s < splits; ++s) {
        const float* part = Jb.part + (int64_t)s * PB * d + j;
#pragma unroll
        for (int c = 0; c < PB; ++c) w[c] += part[(int64_t)c * d];
    }
#pragma unroll
    for (int c = 0; c < PB; ++c) {
        float acc = 0.f;
#pragma unroll
        for (int l = 0; l < PB; ++l) acc += (q_mode ? Ts[c][l] : Ts[l][c]) * w[l];
        Jb.W2[(int64_t)c * d + j] = acc;
    }
}

__global__ __launch_bounds__(256) void qr_init_q_kernel(const QrJob* __restrict__ jobs) {
    const QrJob Jb = jobs[blockIdx.y];
    const int64_t d = Jb.d;
    const int64_t e0 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int64_t e = e0 + q;
        if (e >= d * d) break;
        const int64_t i = e / d, j = e - i * d;
        float val = 0.f;
        if (i == j) val = Jb.Z[i * d + i] < 0.f ? -1.f : 1.f;
        Jb.X[e] = val;
    }
}

__global__ __launch_bounds__(256) void copy_cols_kernel(const CopyJob* __restrict__ jobs) {
    const CopyJob J = jobs[blockIdx.y];
    const int64_t d = J.d, w = J.d - J.c0;
    if (w <= 0) return;
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (e >= d * w) return;
    const int64_t i = e / w, j = J.c0 + (e - i * w);
    J.dst[i * d + j] = J.src[i * d + j];
}

}  // namespace

hipError_t launch_qr_panel(const QrJob* jobs, int njobs, int p, hipStream_t s) {
    if (njobs <= 0) return hipSuccess;
    hipLaunchKernelGGL(qr_panel_kernel, dim3(njobs), dim3(PT), 0, s, jobs, p);
    return hipGetLastError();
}

hipError_t launch_qr_dots(const QrJob* jobs, int njobs, int p, int max_d, int q_mode,
                          hipStream_t s) {
    const int k = p * PB;
    const int L = max_d - k;
    if (njobs <= 0 || L <= 0) return hipSuccess;
    const int ncols = q_mode ? L : L - (L < PB ? L : PB);
    if (ncols <= 0) return hipSuccess;
    dim3 grid((ncols + 511) / 512, qr_splits(L), njobs);
    hipLaunchKernelGGL(qr_dots_kernel, grid, dim3(256), 0, s, jobs, p, q_mode);
    return hipGetLastError();
}

hipError_t launch_qr_reduce(const QrJob* jobs, int njobs, int p, int max_d, int q_mode,
                            hipStream_t s) {
    const int k = p * PB;
    const int L = max_d - k;
    if (njobs <= 0 || L <= 0) return hipSuccess;
    const int ncols = q_mode ? L : L - (L < PB ? L : PB);
    if (ncols <= 0) return hipSuccess;
    hipLaunchKernelGGL(qr_reduce_kernel, dim3((ncols + 255) / 256, njobs), dim3(256), 0, s, jobs, p,
                       q_mode);
    return hipGetLastError();
}

hipError_t launch_qr_init_q(const QrJob* jobs, int njobs, int max_d, hipStream_t s) {
    if (njobs <= 0) return hipSuccess;
    const int64_t n = (int64_t)max_d * max_d;
    hipLaunchKernelGGL(qr_init_q_kernel, dim3((unsigned)((n + 1023) / 1024), njobs), dim3(256), 0, s,
                       jobs);
    return hipGetLastError();
}

hipError_t launch_copy_cols(const CopyJob* jobs, int njobs, int max_d, hipStream_t s) {
    if (njobs <= 0) return hipSuccess;
    const int64_t n = (int64_t)max_d * max_d;
    hipLaunchKernelGGL(copy_cols_kernel, dim3((unsigned)((n + 255) / 256), njobs), dim3(256), 0, s,
                       jobs);
    return hipGetLastError();
}

}  // namespace matopt
