// Blocked Householder QR with explicit Q for the basis refresh (gfx950).
//
// The refresh needs the orthonormal factor Q of Z = QR with diag(R) > 0 for
// d x d inputs up to d = 12288 that are often numerically rank deficient in
// fp32 (products of the Gram matrix with the previous basis). Householder
// reflections keep Q orthonormal to working precision regardless of the
// conditioning of Z, which Cholesky- or Gram-Schmidt-based schemes do not.
//
// Two levels of blocking. Panels of PB = 64 columns are factorised one at a
// time; each updates only the rest of its outer block of NB = 256 columns:
//   1. qr_panel   one 512-thread workgroup per matrix factorises the L x PB
//                 panel in register-resident sub-panels (see below), stores
//                 the reflectors below the diagonal of Z, R on and above it,
//                 and the upper-triangular T of the compact WY form
//                 H_0 ... H_{jb-1} = I - Y T Y^T.
//   2. qr_dots    W = Y^T C for the block's remaining columns C, split over
//                 rows into partial sums (fp32 MFMA 32x32x2 straight from
//                 global memory: both operands read along their contiguous
//                 dimension).
//   3. qr_reduce  sums the partials and applies T^T: W2 = T^T W.
//   4. qr_update  C -= Y W2 on the grouped GEMM tile (unit-lower A loader).
// After the block's panels, the columns right of the block get the block's
// four reflector blocks in one pass on the grouped GEMM (host-side plan):
// Yb = the block's reflectors as an explicit unit-lower matrix
// (qr_copy_block), W = Yb^T C and the Gram matrix S = Yb^T Yb, then W2 by
// block forward substitution (w_q = T_q^T (W_q - sum_{i<q} S_qi w_i), the
// panels' transposed factors applied in order), then C -= Yb W2. The trailing
// matrix is thus read and written once per 256 columns instead of once per
// 64, with K = 256 products.
// Q formation (backward accumulation): X = diag(sign(R_ii)) (qr_init_q, so
// the sign convention costs nothing), then for blocks from last to first
// X[k:, k:] -= Yb W2 with W = Yb^T X[k:, k:] and the backward substitution
// w_q = T_q (W_q - sum_{i>q} S_qi w_i).
//
// Several matrices are factorised in lock step: every launch covers all
// matrices that still have panel p (block b), which are a prefix of the job
// array sorted by d descending.
#include "internal.h"

namespace matopt {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

namespace {

constexpr int PB = kQrPB;
constexpr int PT = kQrPanelThreads;
constexpr int NW = PT / 64;

// ---- panel factorisation -------------------------------------------------
//
// One 512-thread workgroup factorises the L x jb panel (jb <= PB) of one
// matrix. Thread t owns panel rows i = t + 512 r (r < R). The panel is
// processed in sub-panels of SB columns held entirely in registers
// (a[r][c]); a sub-panel is first brought up to date with the reflectors of
// the earlier sub-panels of this panel (left-looking, one SB-wide compact-WY
// block at a time: A -= Y_q (T_q^T (Y_q^T A)), Y_q streamed from memory),
// then factorised column by column without touching memory: per column one
// block reduction for the norm below the diagonal and one for the inner
// products of the new reflector with the other columns of the sub-panel
// (trailing columns: update weights; leading columns: entries of T_q).
// Finally the panel's reflectors are read back once to form their Gram
// matrix S = Y^T Y with fp32 MFMA, and T of the whole panel follows row by
// row from T[c][j] = -tau_j sum_{c<=l<j} T[c][l] S[l][j] (each row depends
// only on itself, so the PB rows need no synchronisation).

constexpr int SLOT = 64;  // values per wavefront in a reduction slot

// Left-looking updates keep a block's reflector rows in registers between
// their two passes when a thread's rows x SB values are at most this many
// (no spills up to 8 rows of 8; one pass instead of two loads from memory:
// an order-3072 orthonormalisation 30.9 -> 30.2 ms).
#ifndef MATOPT_QR_CACHE_Y
#define MATOPT_QR_CACHE_Y 64
#endif

struct PanelShared {
    float red[2][NW][SLOT];
    float Tq[PB][PB + 1];    // sub-panel T blocks on the diagonal (panel-relative indices)
    float P[SLOT];
    float P2[SLOT];
    float tau[PB];
    float alpha;
    float S[PB][PB + 1];     // Gram matrix of the panel's reflectors
    union {
        float gram[NW][32][33];  // per-wavefront partial Gram blocks
        float Tf[PB][PB + 1];    // T of the whole panel
    };
};

// Reduce-scatter of N (power of two, <= 64) values over a wavefront: after
// log2(N) halving exchanges and a butterfly over the remaining lane bits,
// lane l holds the wave sum of value index l >> (6 - log2 N).
template <int N>
__device__ __forceinline__ float rs_reduce(float (&v)[N], int lane, int mask) {
    if constexpr (N == 1) {
        float x = v[0];
        for (int m = mask; m >= 1; m >>= 1) x += __shfl_xor(x, m, 64);
        return x;
    } else {
        float h[N / 2];
        const bool hi = lane & mask;
#pragma unroll
        for (int c = 0; c < N / 2; ++c) {
            const float keep = hi ? v[N / 2 + c] : v[c];
            const float give = hi ? v[c] : v[N / 2 + c];
            h[c] = keep + __shfl_xor(give, mask, 64);
        }
        return rs_reduce<N / 2>(h, lane, mask >> 1);
    }
}

template <int N>
constexpr int ilog2() {
    return N <= 1 ? 0 : 1 + ilog2<N / 2>();
}

// Block sum of N values per thread into sh.red[slot][*][0..N): afterwards
// value c of the block is sum_w sh.red[slot][w][c]. One barrier.
template <int N>
__device__ __forceinline__ void block_partial(float (&v)[N], PanelShared& sh, int slot) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const float x = rs_reduce<N>(v, lane, 32);
    constexpr int shift = 6 - ilog2<N>();
    if ((lane & ((1 << shift) - 1)) == 0) sh.red[slot][wave][lane >> shift] = x;
    __syncthreads();
}

__device__ __forceinline__ float block_value(const PanelShared& sh, int slot, int c) {
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) s += sh.red[slot][w][c];
    return s;
}

struct PanelCtx {
    gmem<float> A;   // top-left of the panel (row k, column k of Z)
    int64_t ld;
    int L;        // rows of the panel
    int jb;       // columns of the panel
    bool vec;     // ld % 4 == 0 and Z 16-byte aligned: groups of 4 columns from a multiple of 4 are 16-byte aligned
};

// Reflector entry Y[i][c] (panel-relative): 0 above the diagonal, 1 on it.
__device__ __forceinline__ float yval(const PanelCtx& c, int i, int col) {
    if (i < col) return 0.f;
    if (i == col) return 1.f;
    return c.A[(int64_t)i * c.ld + col];
}

// Row i's entries at panel columns col0 .. col0 + N - 1 (N a multiple of 4,
// col0 a multiple of 4, all inside the panel, c.vec): N / 4 16-byte loads.
// A thread owns whole rows, so its N values are contiguous; N separate
// 4-byte loads would make every wavefront instruction touch 64 cache lines
// for 4 bytes each.
template <int N>
__device__ __forceinline__ void load_row(const PanelCtx& c, int i, int col0, float (&x)[N]) {
    const gmem<const f32x4> p = (const gmem<const f32x4>)(c.A + (int64_t)i * c.ld + col0);
#pragma unroll
    for (int g = 0; g < N / 4; ++g) {
        const f32x4 v = p[g];
#pragma unroll
        for (int e = 0; e < 4; ++e) x[4 * g + e] = v[e];
    }
}

// Reflector entries Y[i][y0 + l], l < N (as yval), for a block of N
// columns inside the panel.
template <int N>
__device__ __forceinline__ void load_y(const PanelCtx& c, int i, int y0, float (&y)[N]) {
    if (c.vec) {
        load_row<N>(c, i, y0, y);
#pragma unroll
        for (int l = 0; l < N; ++l) y[l] = (i < y0 + l) ? 0.f : (i == y0 + l) ? 1.f : y[l];
    } else {
#pragma unroll
        for (int l = 0; l < N; ++l) y[l] = yval(c, i, y0 + l);
    }
}

template <int R, int SB>
struct SubPanel {
    float a[R][SB];
    int c0;    // first panel column of the sub-panel
    int sbw;   // its width (< SB only in a ragged last panel)
};

// Column J of the current sub-panel (compile-time, so that register indices
// are static). On entry sh.alpha holds its diagonal entry and slot `slot`
// the partial sums of its squared norm below the diagonal.
template <int R, int SB, int J>
__device__ __forceinline__ void column_step(const PanelCtx& c, SubPanel<R, SB>& sp, PanelShared& sh,
                                            int& slot) {
    if (J >= sp.sbw) return;
    const int tid = threadIdx.x;
    const int cj = sp.c0 + J;   // panel row of this column's diagonal

    const float sig = block_value(sh, slot, 0);
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

    // inner products of v_J with the other sub-panel columns
    float part[SB];
#pragma unroll
    for (int q = 0; q < SB; ++q) part[q] = 0.f;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int i = tid + PT * r;
        if (i < c.L && i >= cj) {
            const float vi = (i == cj) ? 1.f : sp.a[r][J] * scale;
#pragma unroll
            for (int q = 0; q < SB; ++q)
                if (q != J) part[q] += vi * sp.a[r][q];
        }
    }
    slot ^= 1;
    block_partial<SB>(part, sh, slot);
    float w[SB];
#pragma unroll
    for (int q = 0; q < SB; ++q) w[q] = (q > J) ? block_value(sh, slot, q) : 0.f;

    // T of the sub-panel, column J (rows < J use the inner products of v_J
    // with the sub-panel's earlier reflectors)
    if (tid < J) {
        float s = 0.f;
        for (int l = tid; l < J; ++l) s += sh.Tq[sp.c0 + tid][sp.c0 + l] * block_value(sh, slot, l);
        sh.Tq[sp.c0 + tid][cj] = -tau * s;
    } else if (tid == J) {
        sh.Tq[cj][cj] = tau;
        sh.tau[cj] = tau;
    }

    // apply H_J, store v_J and beta, and start the next column's norm
    float sig_part = 0.f;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int i = tid + PT * r;
        if (i < c.L && i >= cj) {
            const float vi = (i == cj) ? 1.f : sp.a[r][J] * scale;
#pragma unroll
            for (int q = J + 1; q < SB; ++q) sp.a[r][q] -= tau * vi * w[q];
            sp.a[r][J] = (i == cj) ? beta : vi;
        }
        if constexpr (J + 1 < SB) {
            if (i < c.L) {
                if (i > cj + 1) sig_part += sp.a[r][J + 1] * sp.a[r][J + 1];
                else if (i == cj + 1) sh.alpha = sp.a[r][J + 1];
            }
        }
    }
    if constexpr (J + 1 < SB) {
        float v1[1] = {sig_part};
        slot ^= 1;
        block_partial<1>(v1, sh, slot);
    }
}

template <int R, int SB, int J>
struct SubColumns {
    __device__ __forceinline__ static void run(const PanelCtx& c, SubPanel<R, SB>& sp, PanelShared& sh,
                                               int& slot) {
        column_step<R, SB, J>(c, sp, sh, slot);
        SubColumns<R, SB, J + 1>::run(c, sp, sh, slot);
    }
};
template <int R, int SB>
struct SubColumns<R, SB, SB> {
    __device__ __forceinline__ static void run(const PanelCtx&, SubPanel<R, SB>&, PanelShared&, int&) {}
};

template <int R, int SB>
__global__ __launch_bounds__(PT) void qr_panel_kernel(const QrJob* __restrict__ jobs, int p) {
    __shared__ PanelShared sh;
    const QrJob Jb = jobs[blockIdx.x];
    const int k = p * PB;
    if (k >= Jb.d) return;
    PanelCtx c;
    c.ld = Jb.d;
    c.A = gptr(Jb.Z + (int64_t)k * c.ld + k);
    c.L = Jb.d - k;
    c.jb = min(PB, Jb.d - k);
    c.vec = (Jb.d % 4) == 0 && ((uintptr_t)Jb.Z & 15u) == 0;
    static_assert(SB % 4 == 0, "sub-panels of whole 16-byte groups");
    const int tid = threadIdx.x;
    for (int e = tid; e < PB * (PB + 1); e += PT) (&sh.Tq[0][0])[e] = 0.f;
    int slot = 0;

    SubPanel<R, SB> sp;
    for (int s = 0; s * SB < c.jb; ++s) {
        sp.c0 = s * SB;
        sp.sbw = min(SB, c.jb - sp.c0);
        const bool full = c.vec && sp.sbw == SB;   // whole 16-byte groups inside the panel
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int i = tid + PT * r;
            if (full) {
                if (i < c.L) load_row<SB>(c, i, sp.c0, sp.a[r]);
                else {
#pragma unroll
                    for (int q = 0; q < SB; ++q) sp.a[r][q] = 0.f;
                }
            } else {
#pragma unroll
                for (int q = 0; q < SB; ++q)
                    sp.a[r][q] = (i < c.L && q < sp.sbw) ? c.A[(int64_t)i * c.ld + sp.c0 + q] : 0.f;
            }
        }
        // left-looking: apply the earlier sub-panels' reflector blocks in order
        // (with few rows per thread the block's reflector rows stay in
        // registers between its two passes instead of being loaded twice)
        constexpr bool kCacheY = R * SB <= MATOPT_QR_CACHE_Y;
        for (int qb = 0; qb < s; ++qb) {
            const int y0 = qb * SB;
            float part[SB * SB];
            float yc[kCacheY ? R : 1][SB];
#pragma unroll
            for (int e = 0; e < SB * SB; ++e) part[e] = 0.f;
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const int i = tid + PT * r;
                if (i < c.L && i >= y0) {
                    float y[SB];
                    load_y<SB>(c, i, y0, y);
                    if constexpr (kCacheY) {
#pragma unroll
                        for (int l = 0; l < SB; ++l) yc[r][l] = y[l];
                    }
#pragma unroll
                    for (int l = 0; l < SB; ++l)
#pragma unroll
                        for (int q = 0; q < SB; ++q) part[l * SB + q] += y[l] * sp.a[r][q];
                }
            }
            slot ^= 1;
            block_partial<SB * SB>(part, sh, slot);
            if (tid < SB * SB) sh.P[tid] = block_value(sh, slot, tid);
            __syncthreads();
            if (tid < SB * SB) {   // P2 = T_q^T P
                const int l = tid / SB, q = tid % SB;
                float acc = 0.f;
                for (int m = 0; m <= l; ++m) acc += sh.Tq[y0 + m][y0 + l] * sh.P[m * SB + q];
                sh.P2[tid] = acc;
            }
            __syncthreads();
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const int i = tid + PT * r;
                if (i < c.L && i >= y0) {
                    float y[SB];
                    if constexpr (kCacheY) {
#pragma unroll
                        for (int l = 0; l < SB; ++l) y[l] = yc[r][l];
                    } else {
                        load_y<SB>(c, i, y0, y);
                    }
#pragma unroll
                    for (int q = 0; q < SB; ++q) {
                        float acc = 0.f;
#pragma unroll
                        for (int l = 0; l < SB; ++l) acc += y[l] * sh.P2[l * SB + q];
                        sp.a[r][q] -= acc;
                    }
                }
            }
        }
        // norm of the first column below its diagonal
        {
            float sig_part = 0.f;
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const int i = tid + PT * r;
                if (i < c.L) {
                    if (i > sp.c0) sig_part += sp.a[r][0] * sp.a[r][0];
                    else if (i == sp.c0) sh.alpha = sp.a[r][0];
                }
            }
            float v1[1] = {sig_part};
            slot ^= 1;
            block_partial<1>(v1, sh, slot);
        }
        SubColumns<R, SB, 0>::run(c, sp, sh, slot);
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int i = tid + PT * r;
            if (i < c.L) {
                if (full) {
                    const gmem<f32x4> o = (gmem<f32x4>)(c.A + (int64_t)i * c.ld + sp.c0);
#pragma unroll
                    for (int g = 0; g < SB / 4; ++g)
                        o[g] = (f32x4){sp.a[r][4 * g], sp.a[r][4 * g + 1], sp.a[r][4 * g + 2], sp.a[r][4 * g + 3]};
                } else {
#pragma unroll
                    for (int q = 0; q < SB; ++q)
                        if (q < sp.sbw) c.A[(int64_t)i * c.ld + sp.c0 + q] = sp.a[r][q];
                }
            }
        }
        __syncthreads();   // stored reflectors visible to the next sub-panel's loads; T_q complete
    }

    // Gram S = Y^T Y of the panel's reflectors (PB x PB) as 32x32 fp32 MFMA
    // blocks: lane l of wave w supplies Y[row + l/32][32 b + l%32] as the
    // operand of column block b. Eight row pairs are loaded before their
    // MFMAs are issued.
    {
        constexpr int NB = PB / 32;
        constexpr int U = 8;
        const int lane = tid & 63, wave = tid >> 6, h = lane >> 5, l32 = lane & 31;
        f32x16 acc[NB][NB];
#pragma unroll
        for (int bi = 0; bi < NB; ++bi)
#pragma unroll
            for (int bj = 0; bj < NB; ++bj)
#pragma unroll
                for (int e = 0; e < 16; ++e) acc[bi][bj][e] = 0.f;
        const int rows_per = ((c.L + NW - 1) / NW + 1) & ~1;
        const int r0 = wave * rows_per, r1 = min(c.L, r0 + rows_per);
        for (int i0 = r0; i0 < r1; i0 += 2 * U) {
            float y[U][NB];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int row = i0 + 2 * u + h;
#pragma unroll
                for (int b = 0; b < NB; ++b) {
                    const int col = 32 * b + l32;
                    y[u][b] = (row < r1 && col < c.jb) ? yval(c, row, col) : 0.f;
                }
            }
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int bi = 0; bi < NB; ++bi)
#pragma unroll
                    for (int bj = 0; bj < NB; ++bj)
                        acc[bi][bj] = __builtin_amdgcn_mfma_f32_32x32x2f32(y[u][bi], y[u][bj], acc[bi][bj], 0, 0, 0);
        }
#pragma unroll
        for (int bi = 0; bi < NB; ++bi)
#pragma unroll
            for (int bj = 0; bj < NB; ++bj) {
#pragma unroll
                for (int e = 0; e < 16; ++e) sh.gram[wave][8 * (e >> 2) + 4 * h + (e & 3)][l32] = acc[bi][bj][e];
                __syncthreads();
                for (int e = tid; e < 32 * 32; e += PT) {
                    const int i = e / 32, j = e % 32;
                    float sum = 0.f;
#pragma unroll
                    for (int w = 0; w < NW; ++w) sum += sh.gram[w][i][j];
                    sh.S[32 * bi + i][32 * bj + j] = sum;
                }
                __syncthreads();
            }
    }
    if (tid < PB) {
        const int r = tid;
        for (int j = 0; j < PB; ++j) {
            float v = 0.f;
            if (r < c.jb && j < c.jb && j >= r) {
                if (j == r) {
                    v = sh.tau[r];
                } else {
                    float sum = 0.f;
                    for (int l = r; l < j; ++l) sum += sh.Tf[r][l] * sh.S[l][j];
                    v = -sh.tau[j] * sum;
                }
            }
            sh.Tf[r][j] = v;
        }
    }
    __syncthreads();
    gmem<float> Tout = gptr(Jb.T + (int64_t)p * PB * PB);
    for (int e = tid; e < PB * PB; e += PT) Tout[e] = sh.Tf[e / PB][e % PB];
}

// Partial products W_s = Y[rows of split s]^T C[rows of split s].
// A wavefront owns a PB x 128 block of W (PB/32 x 4 MFMA accumulators that
// share operands); lane l supplies Y[row + l/32][32 b + l%32] and
// C[row + l/32][col + l%32], i.e. 128-byte row segments of both matrices.
__global__ __launch_bounds__(256) void qr_dots_kernel(const QrJob* __restrict__ jobs, QrClasses cls,
                                                     int p) {
    constexpr int NB = PB / 32;
    int job, local;
    if (!qr_locate(cls, QG_DOTS, p, blockIdx.x, job, local)) return;
    const QrJob Jb = jobs[job];
    const int k = p * PB;
    const int d = Jb.d;
    const int jb = min(PB, d - k), L = d - k;
    const int ncols = qr_inblock_cols(d, p);
    const int splits = qr_splits(L), kc = qr_chunk(L, splits);
    const int nxb = (ncols + 511) / 512;
    const int s = local / nxb;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, h = lane >> 5, l32 = lane & 31;
    const int j0 = (local % nxb) * 512 + wave * 128;
    if (j0 >= ncols) return;
    const int r0 = s * kc, r1 = min(L, r0 + kc);
    gmem<const float> Y = gptr((const float*)Jb.Z + (int64_t)k * d + k);
    gmem<const float> C = gptr((const float*)Jb.Z + (int64_t)k * d + k + jb);

    f32x16 acc[NB][4];
#pragma unroll
    for (int a = 0; a < NB; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;

    // Four row pairs per iteration; the next iteration's rows are loaded
    // before this one's MFMAs, so the loads' latency overlaps them.
    constexpr int U = 4;
    float y[U][NB], x[U][4], yn[U][NB], xn[U][4];
    auto load = [&](int i0, float (&yy)[U][NB], float (&xx)[U][4]) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int row = i0 + 2 * u + h;
#pragma unroll
            for (int a = 0; a < NB; ++a) yy[u][a] = 0.f;
#pragma unroll
            for (int b = 0; b < 4; ++b) xx[u][b] = 0.f;
            if (row < r1) {
#pragma unroll
                for (int a = 0; a < NB; ++a) {
                    const int yc = 32 * a + l32;
                    if (yc < jb) yy[u][a] = row < yc ? 0.f : (row == yc ? 1.f : Y[(int64_t)row * d + yc]);
                }
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    const int col = j0 + 32 * b + l32;
                    if (col < ncols) xx[u][b] = C[(int64_t)row * d + col];
                }
            }
        }
    };
    load(r0, y, x);
    for (int i0 = r0; i0 < r1; i0 += 2 * U) {
        if (i0 + 2 * U < r1) load(i0 + 2 * U, yn, xn);
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int a = 0; a < NB; ++a)
#pragma unroll
                for (int b = 0; b < 4; ++b)
                    acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x2f32(y[u][a], x[u][b], acc[a][b], 0, 0, 0);
#pragma unroll
        for (int u = 0; u < U; ++u) {
#pragma unroll
            for (int a = 0; a < NB; ++a) y[u][a] = yn[u][a];
#pragma unroll
            for (int b = 0; b < 4; ++b) x[u][b] = xn[u][b];
        }
    }

    // split s's partials: PB rows of kQrPartLd (the in-block columns) floats
    static_assert(kQrPartLd >= kQrNB - PB, "the in-block columns fit in a partial row");
    gmem<float> part = gptr(Jb.part + (int64_t)s * PB * kQrPartLd);
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        const int j = j0 + 32 * b + l32;
        if (j >= ncols) continue;
#pragma unroll
        for (int a = 0; a < NB; ++a)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int cc = 32 * a + 8 * (r >> 2) + 4 * h + (r & 3);
                part[(int64_t)cc * kQrPartLd + j] = acc[a][b][r];
            }
    }
}

// W2[:, j] = T^T (sum_s W_s[:, j]), 64 columns j per workgroup (kQrReduceCols):
// the 256 threads first add up the split partials of the 64 x 64 block (16
// sums each, loads coalesced along j) into LDS, then the thread of column j
// in wavefront g forms outputs c = 16 g .. 16 g + 15, reading T rows as LDS
// broadcasts. Spreading a job's columns over several workgroups this way
// keeps the partials' loads from queueing on one CU.
__global__ __launch_bounds__(256) void qr_reduce_kernel(const QrJob* __restrict__ jobs, QrClasses C, int p) {
    constexpr int JC = kQrReduceCols;
    static_assert(JC == 64 && PB == 64, "four wavefronts of 64 columns, 16 of the 64 rows each");
    __shared__ __attribute__((aligned(16))) float Ts[PB][PB];
    __shared__ float Ws[PB][JC + 1];
    int job, local;
    if (!qr_locate(C, QG_REDUCE, p, blockIdx.x, job, local)) return;
    const QrJob Jb = jobs[job];
    const int k = p * PB;
    const int d = Jb.d;
    const int L = d - k;
    const int ncols = qr_inblock_cols(d, p);
    const int tid = threadIdx.x, jj = tid & 63, g = tid >> 6;
    const int j = local * JC + jj;
    gmem<const float> Tp = gptr((const float*)Jb.T + (int64_t)p * PB * PB);
    for (int e = tid; e < PB * PB; e += 256) Ts[e / PB][e % PB] = Tp[e];
    const int splits = qr_splits(L);
    float w[16];
#pragma unroll
    for (int c = 0; c < 16; ++c) w[c] = 0.f;
    if (j < ncols) {
        for (int s = 0; s < splits; ++s) {
            gmem<const float> part = gptr((const float*)Jb.part + ((int64_t)s * PB + 16 * g) * kQrPartLd + j);
#pragma unroll
            for (int c = 0; c < 16; ++c) w[c] += part[(int64_t)c * kQrPartLd];
        }
    }
#pragma unroll
    for (int c = 0; c < 16; ++c) Ws[16 * g + c][jj] = w[c];
    __syncthreads();
    if (j >= ncols) return;
    float acc[16];
#pragma unroll
    for (int c = 0; c < 16; ++c) acc[c] = 0.f;
#pragma unroll 4
    for (int l = 0; l < PB; ++l) {
        const float x = Ws[l][jj];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const f32x4 t = *(const f32x4*)&Ts[l][16 * g + 4 * q];
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[4 * q + e] += t[e] * x;
        }
    }
#pragma unroll
    for (int c = 0; c < 16; ++c) gptr(Jb.W2)[(int64_t)(16 * g + c) * d + j] = acc[c];
}

// The helper copies below move 16-byte groups of four consecutive columns
// when a row's length and the base addresses allow it (else one float at a
// time), in a grid-stride loop over each job's groups: the grid is sized for
// the largest job, and smaller jobs' workgroups leave the loop early.

__device__ __forceinline__ bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// X = diag(sign Z_ii): the start of the backward accumulation of Q.
__global__ __launch_bounds__(256) void qr_init_q_kernel(const QrJob* __restrict__ jobs) {
    const QrJob Jb = jobs[blockIdx.y];
    const int64_t d = Jb.d;
    const int64_t stride = (int64_t)gridDim.x * 256;
    const gmem<const float> Z = gptr((const float*)Jb.Z);
    if (d % 4 == 0 && aligned16(Jb.X)) {
        const gmem<f32x4> X = (gmem<f32x4>)Jb.X;
        for (int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x; g < d * d / 4; g += stride) {
            const int64_t i = (4 * g) / d, j0 = 4 * g - i * d;
            f32x4 v = {0.f, 0.f, 0.f, 0.f};
            if (i >= j0 && i < j0 + 4) v[i - j0] = Z[i * d + i] < 0.f ? -1.f : 1.f;
            X[g] = v;
        }
    } else {
        for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < d * d; e += stride) {
            const int64_t i = e / d, j = e - i * d;
            gptr(Jb.X)[e] = (i == j) ? (Z[i * d + i] < 0.f ? -1.f : 1.f) : 0.f;
        }
    }
}

// Columns [c0, d) of src into dst (both d x d, row stride d).
__global__ __launch_bounds__(256) void copy_cols_kernel(const CopyJob* __restrict__ jobs) {
    const CopyJob J = jobs[blockIdx.y];
    const int64_t d = J.d, w = J.d - J.c0;
    if (w <= 0) return;
    const int64_t stride = (int64_t)gridDim.x * 256;
    if (d % 4 == 0 && J.c0 % 4 == 0 && aligned16(J.src) && aligned16(J.dst)) {
        const int64_t gw = w / 4;   // groups per row
        for (int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x; g < d * gw; g += stride) {
            const int64_t i = g / gw, j = J.c0 + 4 * (g - i * gw);
            *(gmem<f32x4>)(J.dst + i * d + j) = *(const gmem<const f32x4>)(J.src + i * d + j);
        }
    } else {
        for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < d * w; e += stride) {
            const int64_t i = e / w, j = J.c0 + (e - i * w);
            gptr(J.dst)[i * d + j] = gptr(J.src)[i * d + j];
        }
    }
}

// Yb[i][c] = Y[kB + i][kB + c] of outer block b as a unit-lower matrix
// (zeros above the diagonal, ones on it, the stored reflectors below), for
// i < d - kB and c < NB; columns past the matrix are zero.
__global__ __launch_bounds__(256) void qr_copy_block_kernel(const QrJob* __restrict__ jobs, int b) {
    const QrJob J = jobs[blockIdx.y];
    const int kB = b * kQrNB;
    const int64_t d = J.d, L = d - kB;
    if (L <= 0) return;
    const int64_t stride = (int64_t)gridDim.x * 256;
    const gmem<const float> Z = gptr((const float*)J.Z);
    auto yv = [&](int64_t i, int c, float z) { return kB + c >= d ? 0.f : i == c ? 1.f : i > c ? z : 0.f; };
    if (d % 4 == 0 && aligned16(J.Z) && aligned16(J.Yb)) {
        constexpr int GR = kQrNB / 4;   // groups per row of Yb
        const gmem<f32x4> Yb = (gmem<f32x4>)J.Yb;
        for (int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x; g < L * GR; g += stride) {
            const int64_t i = g / GR;
            const int c0 = 4 * (int)(g - i * GR);
            // kB, c0 and d are multiples of 4: a group lies wholly inside the
            // matrix's columns or wholly past them
            f32x4 z = {0.f, 0.f, 0.f, 0.f};
            if (kB + c0 < d && i > c0) z = *(const gmem<const f32x4>)(J.Z + (kB + i) * d + kB + c0);
            f32x4 v;
#pragma unroll
            for (int q = 0; q < 4; ++q) v[q] = yv(i, c0 + q, z[q]);
            Yb[g] = v;
        }
    } else {
        for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < L * kQrNB; e += stride) {
            const int64_t i = e / kQrNB;
            const int c = (int)(e - i * kQrNB);
            const float z = (kB + c < d && i > c) ? Z[(kB + i) * d + kB + c] : 0.f;
            gptr(J.Yb)[e] = yv(i, c, z);
        }
    }
}

// ---- tall panels: rows spread over many workgroups ---------------------
//
// One workgroup factorises a panel of L rows by streaming its column block
// through one CU once per column (plus the left-looking passes), so a few
// tall panels leave most of the GPU idle. Here a panel's rows are split into
// slices of kQrTallRows, one workgroup each, over all active matrices at
// once, in one cooperative launch (every workgroup resident, which the
// runtime checks): each workgroup keeps its slice in LDS for the whole panel,
// and the columns advance in lock step with one grid-wide barrier per
// column.
//
// Column j: every workgroup of a matrix sums the partial column sums its
// slices left (in a fixed slice order, so all of them, in every run, get the
// same values), forms the reflector of column j from alpha = A[j][j] and
// sigma = sum_{i > j} A[i][j]^2 exactly as qr_panel_kernel does, and the
// update weights w_q = v_j^T A[:, q] = A[j][q] + scale sum_{i > j} A[i][j]
// A[i][q]; it applies H_j to its rows (A[i][q] -= tau v_i w_q, q > j),
// stores v below the diagonal and beta on it, and leaves the partial sums of
// column j + 1 over its rows below j + 1 (A[i][j+1] A[i][q], q >= j + 1, from
// the updated values) and, in the workgroup holding row j + 1, that row. The
// pass before column 0 only leaves column 0's sums. Thread t handles column
// q = t mod 64 of the slice rows rg + 4 r (rg = t / 64, one wavefront each);
// a wavefront reads a row's column-j and column-(j+1) entries, which its own
// lanes j and j+1 rewrite, with the same instructions before any lane stores.
// At the end each workgroup writes its rows back and the Gram block of its
// slice of the reflectors; qr_tall_t_kernel forms T.
//
// The barrier: thread 0 of each workgroup adds one to a counter with release
// semantics and waits, with acquire semantics, for the count of all
// workgroups; the sums cross workgroups (and XCDs) through agent-scope atomic
// stores and loads. Every wait is bounded: past about a quarter second the
// workgroup raises the error flag, stops waiting (so the grid always drains)
// and qr_tall_t_kernel turns that panel's T into NaN, so a failure shows in
// the results instead of hanging the device.
//
// Scratch in the job's `part` buffer (floats; gmax = slices of the whole
// order d): the partial sums [2][gmax][64] (ping-pong by column parity), the
// diagonal row [2][64], tau [64], the per-slice Gram blocks [gmax][64][64],
// then the barrier counter and error flag (the first job's are used).

__host__ __device__ inline int qr_tall_gmax(int d) { return (d + kQrTallRows - 1) / kQrTallRows; }

struct TallScratch {
    float* sums;   // [2][gmax][64]
    float* row;    // [2][64]
    float* tau;    // [64]
    float* gram;   // [gmax][64][64]
    unsigned* bar; // [0] counter, [1] error flag
    __device__ TallScratch(const QrJob& J) {
        const int gmax = qr_tall_gmax(J.d);
        sums = J.part;
        row = sums + 2 * gmax * 64;
        tau = row + 128;
        gram = tau + 64;
        bar = (unsigned*)(gram + (int64_t)gmax * PB * PB);
    }
};

__device__ __forceinline__ void coop_barrier(unsigned* bar, unsigned target) {
    __syncthreads();
    if (threadIdx.x == 0) {
        __hip_atomic_fetch_add(bar, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
        unsigned spins = 0;
        while (__hip_atomic_load(bar, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT) < target &&
               __hip_atomic_load(bar + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0u) {
            __builtin_amdgcn_s_sleep(2);
            if (++spins == (1u << 22)) {
                __hip_atomic_store(bar + 1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                break;
            }
        }
    }
    __syncthreads();
}

__device__ __forceinline__ void st_agent(float* p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_agent(const float* p) {
    return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__global__ __launch_bounds__(256) void qr_coop_panel_kernel(const QrJob* __restrict__ jobs, QrClasses cls, int p,
                                                            int nblocks) {
    __shared__ float As[kQrTallRows][PB];
    __shared__ float sD[64], sRow[64], red[4][64];
    int job = 0, slice = 0;
    const bool have = qr_locate(cls, QG_TALL, p, blockIdx.x, job, slice);
    const QrJob Jb = jobs[job];
    const int d = Jb.d, k = p * PB, L = d - k, jb = have ? min(PB, L) : 0;
    const int G = (L + kQrTallRows - 1) / kQrTallRows;
    const TallScratch sc(Jb);
    unsigned* bar = TallScratch(jobs[0]).bar;
    const int gmax = qr_tall_gmax(d);
    const int tid = threadIdx.x, q = tid & 63, rg = tid >> 6;
    gmem<float> A = gptr(Jb.Z + (int64_t)k * d + k);
    const int r0 = slice * kQrTallRows;
    const int rows = have ? min(L - r0, kQrTallRows) : 0;

    for (int e = tid; e < kQrTallRows * PB; e += 256) {
        const int r = e / PB, c = e % PB;
        As[r][c] = (r < rows && c < jb) ? A[(int64_t)(r0 + r) * d + c] : 0.f;
    }
    __syncthreads();

    unsigned nb = 0;
    for (int j = -1; j < PB; ++j) {
        if (j >= 0) coop_barrier(bar, (unsigned)nblocks * ++nb);
        if (j >= jb) continue;   // this matrix's last panel is narrower: idle, but in every barrier
        float beta = 0.f, tau = 0.f, scale = 0.f, w = 0.f, w1 = 0.f;
        if (j >= 0) {
            // the slices' partial sums of column j: the four wavefronts load
            // every fourth slice at once (all loads in flight together), then
            // the four sums are added in a fixed order
            {
                const float* in = sc.sums + (j & 1) * gmax * 64 + q;
                float part[12];
#pragma unroll
                for (int u = 0; u < 12; ++u) {
                    const int g = rg + 4 * u;
                    part[u] = g < G ? ld_agent(in + g * 64) : 0.f;
                }
                float sum = 0.f;
#pragma unroll
                for (int u = 0; u < 12; ++u) sum += part[u];
                for (int g = rg + 48; g < G; g += 4) sum += ld_agent(in + g * 64);   // orders past 12288
                red[rg][q] = sum;
                if (rg == 0) sRow[q] = ld_agent(sc.row + (j & 1) * 64 + q);
            }
            __syncthreads();
            if (tid < 64) sD[tid] = red[0][tid] + red[1][tid] + red[2][tid] + red[3][tid];
            __syncthreads();
            const float alpha = sRow[j], sig = sD[j];
            if (sig == 0.f) {
                beta = alpha;
            } else {
                const float nrm = __builtin_sqrtf(alpha * alpha + sig);
                beta = -__builtin_copysignf(nrm, alpha);
                tau = (beta - alpha) / beta;
                scale = 1.f / (alpha - beta);
            }
            if (q > j && q < jb) w = sRow[q] + scale * sD[q];
            if (j + 1 < jb) w1 = sRow[j + 1] + scale * sD[j + 1];
            if (slice == 0 && tid == 0) gptr(sc.tau)[j] = tau;
        }
        const int jn = j + 1;   // the column whose sums this pass leaves
        const bool next = jn < jb;
        const bool qn = next && q >= jn && q < jb;
        const int lo = j < 0 ? 0 : j;   // rows above column j's diagonal are not touched
        float acc = 0.f;
        constexpr int U = 8;   // rows of a wavefront in flight
        for (int rb = rg; rb < rows; rb += 4 * U) {
            float aj[U], a1o[U], aq[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int r = min(rb + 4 * u, kQrTallRows - 1);
                aj[u] = j >= 0 ? As[r][j] : 0.f;
                a1o[u] = next ? As[r][jn] : 0.f;
                aq[u] = As[r][q];
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int r = rb + 4 * u, i = r0 + r;
                if (r >= rows || i < lo) continue;
                float anew = aq[u], a1 = a1o[u];
                if (j >= 0) {
                    const float vi = (i == j) ? 1.f : scale * aj[u];
                    a1 = a1o[u] - tau * vi * w1;
                    if (q > j && q < jb) anew = aq[u] - tau * vi * w;
                    if (q > j) As[r][q] = anew;
                    else if (q == j) As[r][j] = (i == j) ? beta : vi;
                }
                if (qn) {
                    if (i > jn) acc += a1 * anew;
                    else if (i == jn) st_agent(sc.row + (jn & 1) * 64 + q, anew);
                }
            }
        }
        if (!next) continue;
        __syncthreads();   // red[] was read for this column's sums above
        red[rg][q] = acc;
        __syncthreads();
        if (tid < 64) {
            const float sum = red[0][tid] + red[1][tid] + red[2][tid] + red[3][tid];
            st_agent(sc.sums + (jn & 1) * gmax * 64 + slice * 64 + tid, sum);
        }
    }
    __syncthreads();
    // the factorised slice back to Z, and the slice's Gram block of Y
    for (int e = tid; e < rows * PB; e += 256) {
        const int r = e / PB, c = e % PB;
        if (c < jb) A[(int64_t)(r0 + r) * d + c] = As[r][c];
    }
    if (!have) return;
    const int bl = tid / 16, bm = tid % 16;
    float g[4][4] = {};
    for (int r = 0; r < rows; ++r) {
        const int i = r0 + r;
        float yl[4], ym[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int cl = 4 * bl + e, cm = 4 * bm + e;
            yl[e] = (cl >= jb || i < cl) ? 0.f : (i == cl ? 1.f : As[r][cl]);
            ym[e] = (cm >= jb || i < cm) ? 0.f : (i == cm ? 1.f : As[r][cm]);
        }
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int b = 0; b < 4; ++b) g[a][b] += yl[a] * ym[b];
    }
    gmem<float> out = gptr(sc.gram + (int64_t)slice * PB * PB);
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) out[(4 * bl + a) * PB + 4 * bm + b] = g[a][b];
}

__global__ void qr_coop_reset_kernel(const QrJob* __restrict__ jobs) {
    unsigned* bar = TallScratch(jobs[0]).bar;
    if (threadIdx.x < 2) bar[threadIdx.x] = 0u;
}

// T of the panel from the summed Gram blocks and tau, one workgroup per job,
// by the recurrence of qr_panel_kernel: T[c][j] = -tau_j sum_{c<=l<j} T[c][l]
// S[l][j], tau on the diagonal.
__global__ __launch_bounds__(256) void qr_tall_t_kernel(const QrJob* __restrict__ jobs, int p) {
    __shared__ float S[PB][PB + 1], Tf[PB][PB + 1], tau[PB];
    const QrJob Jb = jobs[blockIdx.x];
    const int d = Jb.d, k = p * PB;
    if (k >= d) return;
    const int L = d - k, jb = min(PB, L);
    const int G = (L + kQrTallRows - 1) / kQrTallRows;
    const TallScratch sc(Jb);
    for (int e = threadIdx.x; e < PB * PB; e += 256) {
        gmem<const float> g = gptr((const float*)sc.gram + e);
        float sum = 0.f;
        for (int s = 0; s < G; ++s) sum += g[(int64_t)s * PB * PB];
        S[e / PB][e % PB] = sum;
    }
    if (threadIdx.x < PB) tau[threadIdx.x] = threadIdx.x < jb ? gptr((const float*)sc.tau)[threadIdx.x] : 0.f;
    // a barrier that gave up (the error flag): make the failure visible
    const bool failed = gptr((const unsigned*)TallScratch(jobs[0]).bar)[1] != 0u;
    __syncthreads();
    if (threadIdx.x < PB) {
        const int r = threadIdx.x;
        for (int j = 0; j < PB; ++j) {
            float v = 0.f;
            if (r < jb && j < jb && j >= r) {
                if (j == r) {
                    v = tau[r];
                } else {
                    float sum = 0.f;
                    for (int l = r; l < j; ++l) sum += Tf[r][l] * S[l][j];
                    v = -tau[j] * sum;
                }
            }
            Tf[r][j] = v;
        }
    }
    __syncthreads();
    gmem<float> Tout = gptr(Jb.T + (int64_t)p * PB * PB);
    for (int e = threadIdx.x; e < PB * PB; e += 256) Tout[e] = failed ? __builtin_nanf("") : Tf[e / PB][e % PB];
}

}  // namespace

// Workgroups per job of the helper copies for at most n elements: about four
// 16-byte groups per thread.
unsigned helper_blocks(int64_t n) {
    const int64_t groups = (n + 3) / 4;
    return (unsigned)std::max<int64_t>(1, (groups + 4 * 256 - 1) / (4 * 256));
}

hipError_t launch_qr_copy_block(const QrJob* jobs, int njobs, int b, int max_d, hipStream_t s) {
    const int64_t L = (int64_t)max_d - (int64_t)b * kQrNB;
    if (njobs <= 0 || L <= 0) return hipSuccess;
    hipLaunchKernelGGL(qr_copy_block_kernel, dim3(helper_blocks(L * kQrNB), njobs), dim3(256), 0, s, jobs, b);
    return hipGetLastError();
}

hipError_t launch_qr_panel(const QrJob* jobs, int njobs, int p, int max_d, hipStream_t s) {
    const int L = max_d - p * PB;
    if (njobs <= 0 || L <= 0) return hipSuccess;
    const int rows = (L + PT - 1) / PT;
    dim3 g(njobs), b(PT);
    if (rows <= 1)       qr_panel_kernel<1, 8><<<g, b, 0, s>>>(jobs, p);
    else if (rows <= 2)  qr_panel_kernel<2, 8><<<g, b, 0, s>>>(jobs, p);
    else if (rows <= 4)  qr_panel_kernel<4, 8><<<g, b, 0, s>>>(jobs, p);
    else if (rows <= 6)  qr_panel_kernel<6, 8><<<g, b, 0, s>>>(jobs, p);
    else if (rows <= 8)  qr_panel_kernel<8, 8><<<g, b, 0, s>>>(jobs, p);
    else if (rows <= 12) qr_panel_kernel<12, 8><<<g, b, 0, s>>>(jobs, p);
    else if (rows <= 16) qr_panel_kernel<16, 4><<<g, b, 0, s>>>(jobs, p);
    else if (rows <= 24) qr_panel_kernel<24, 4><<<g, b, 0, s>>>(jobs, p);
    else if (rows <= 32) qr_panel_kernel<32, 4><<<g, b, 0, s>>>(jobs, p);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

// Workgroups of the cooperative panel kernel that can be resident at once
// on the current device (0 if the runtime cannot launch it cooperatively).
int qr_coop_capacity() {
    static int cached[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    if (cached[dev]) return cached[dev] > 0 ? cached[dev] : 0;
    int coop = 0, cus = 0, per = 0;
    if (hipDeviceGetAttribute(&coop, hipDeviceAttributeCooperativeLaunch, dev) != hipSuccess || !coop ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, qr_coop_panel_kernel, 256, 0) != hipSuccess) {
        cached[dev] = -1;
        return 0;
    }
    cached[dev] = cus * per > 0 ? cus * per : -1;
    return cached[dev] > 0 ? cached[dev] : 0;
}

int qr_tall_blocks(const std::vector<QrClasses>& C, int p) {
    if (C.size() != 1) return -1;   // one launch covers one set of classes
    return qr_total_blocks(C[0], QG_TALL, p);
}

hipError_t launch_qr_panel_tall(const QrJob* jobs, int njobs, const std::vector<QrClasses>& C, int p, int max_d,
                                hipStream_t s) {
    const int L = max_d - p * PB;
    if (njobs <= 0 || L <= 0) return hipSuccess;
    int blocks = qr_tall_blocks(C, p);
    if (blocks <= 0 || blocks > qr_coop_capacity()) return hipErrorInvalidValue;
    hipLaunchKernelGGL(qr_coop_reset_kernel, dim3(1), dim3(64), 0, s, jobs);
    QrClasses c = C[0];
    void* args[] = {(void*)&jobs, (void*)&c, (void*)&p, (void*)&blocks};
    hipError_t e = hipLaunchCooperativeKernel((const void*)qr_coop_panel_kernel, dim3(blocks), dim3(256), args, 0, s);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(qr_tall_t_kernel, dim3(njobs), dim3(256), 0, s, jobs, p);
    return hipGetLastError();
}

hipError_t launch_qr_dots(const QrJob* jobs, const QrClasses& C, int p, hipStream_t s) {
    const int blocks = qr_total_blocks(C, QG_DOTS, p);
    if (blocks <= 0) return hipSuccess;
    hipLaunchKernelGGL(qr_dots_kernel, dim3(blocks), dim3(256), 0, s, jobs, C, p);
    return hipGetLastError();
}

hipError_t launch_qr_reduce(const QrJob* jobs, const QrClasses& C, int p, hipStream_t s) {
    const int blocks = qr_total_blocks(C, QG_REDUCE, p);
    if (blocks <= 0) return hipSuccess;
    hipLaunchKernelGGL(qr_reduce_kernel, dim3(blocks), dim3(256), 0, s, jobs, C, p);
    return hipGetLastError();
}

hipError_t launch_qr_init_q(const QrJob* jobs, int njobs, int max_d, hipStream_t s) {
    if (njobs <= 0) return hipSuccess;
    const int64_t n = (int64_t)max_d * max_d;
    hipLaunchKernelGGL(qr_init_q_kernel, dim3(helper_blocks(n), njobs), dim3(256), 0, s, jobs);
    return hipGetLastError();
}

hipError_t launch_copy_cols(const CopyJob* jobs, int njobs, int max_d, hipStream_t s) {
    if (njobs <= 0) return hipSuccess;
    const int64_t n = (int64_t)max_d * max_d;
    hipLaunchKernelGGL(copy_cols_kernel, dim3(helper_blocks(n), njobs), dim3(256), 0, s, jobs);
    return hipGetLastError();
}

}  // namespace matopt
