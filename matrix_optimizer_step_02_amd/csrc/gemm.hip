// Grouped fp32 MFMA GEMM for gfx950 (CDNA4).
//
// Serves the two-sided rotations U^T X V, the rotation back U u V^T (with the
// weight update fused into the epilogue), the Gram products of the basis
// refresh, and the compact-WY trailing updates of the blocked QR.
//
// gfx950 has no reduced-precision fp32 matrix path, so the contraction runs on
// v_mfma_f32_32x32x2_f32 (32x32 outputs, 2-deep k, fp32 accumulate). A tile
// configuration Cfg<WAVES_M, WAVES_N, BLK_M, BLK_N> gives each wavefront a
// (32 BLK_M) x (32 BLK_N) block of the output held as BLK_M x BLK_N MFMA
// accumulators, and the workgroup WAVES_M x WAVES_N wavefronts. K advances in
// slabs of 32 staged through LDS with two buffers, so one barrier per slab
// separates the fill of slab k+1 from the reads of slab k.
//
// Operand staging. An fp32 operand goes from global memory straight into LDS
// (global_load_lds: each wavefront instruction writes 64 lanes x 16 bytes to
// one contiguous kilobyte of LDS, in lane order), so it takes no registers and
// no LDS store instructions; the fill of slab k+1 is issued before the MFMAs
// of slab k. Addresses are clamped into the operand, so rows and columns past
// the edge hold copies of valid data that only reach outputs that are never
// stored; k values past K are zeroed in LDS afterwards (only a last, partial
// slab has any). A bf16 operand is loaded into registers, widened and masked,
// and stored to the same LDS layout after the MFMAs.
//
// LDS layouts, unpadded, with every MFMA operand read conflict-free:
//  * an operand whose non-k index is contiguous in memory (A stored K x M,
//    B stored K x N) is kept k-major, [32][BM or BN], read 4 bytes per lane
//    with 32 consecutive lanes on consecutive words;
//  * an operand whose k index is contiguous (A stored M x K, B stored N x K)
//    is kept [BM or BN][32], read 16 bytes per lane. Within a group of 8 k
//    values, MFMA s (0..3) takes k = 8g + s from lanes 0..31 and k = 8g + 4 + s
//    from lanes 32..63, so one 16-byte read feeds four MFMAs. The 16-byte
//    group q of row r is stored at slot q ^ swz(r), swz(r) = (r + r/8) mod 8,
//    which puts any 8 aligned consecutive rows, and the rows of one parity
//    among any 16 aligned consecutive rows, on distinct slots.
// The same k assignment is used for both operands, so the sum is unchanged.
//
// Work distribution: one workgroup per output tile; problems of a grouped
// launch are concatenated in tile space in longest-processing-time order
// (costliest k first) by the host. Consecutive workgroup ids are spread by
// the dispatcher over the 8 XCDs, so ids are remapped in windows of
// 8 x XCD_RUN tiles to give each XCD XCD_RUN neighbouring tiles (shared A
// rows / B columns in its own L2) while keeping the LPT order at window
// granularity.
#include "internal.h"

namespace matopt {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

namespace {

#ifndef MATOPT_XCD_RUN
#define MATOPT_XCD_RUN 16
#endif
#ifndef MATOPT_GROUP_M
#define MATOPT_GROUP_M 4
#endif
constexpr int XCD = 8;
constexpr int XCD_RUN = MATOPT_XCD_RUN;
constexpr int GROUP_M = MATOPT_GROUP_M;

template <int WAVES_M, int WAVES_N, int BLK_M, int BLK_N, int SLAB_K = 32>
struct Cfg {
    static constexpr int WM = WAVES_M, WN = WAVES_N, TM = BLK_M, TN = BLK_N;
    static constexpr int BK = SLAB_K;   // k values per LDS slab
    static_assert(BK == 16 || BK == 32, "slabs of 16 or 32 k values (4 or 8 groups of 4 per row)");
    static constexpr int NT = 64 * WAVES_M * WAVES_N;
    static constexpr int BM = 32 * BLK_M * WAVES_M;
    static constexpr int BN = 32 * BLK_N * WAVES_N;
    static constexpr int QA = BM * BK / 4 / NT;   // float4 loads of A per thread per slab
    static constexpr int QB = BN * BK / 4 / NT;
    static constexpr int AS = BM * BK;   // floats of one A buffer (either layout)
    static constexpr int BS = BN * BK;
    static constexpr int SMEM = 2 * (AS + BS);
    static constexpr int NW = NT / 64;
    static constexpr int CA = AS / 256 / NW;   // kilobyte LDS chunks of A filled per wavefront per slab
    static constexpr int CB = BS / 256 / NW;
    static_assert(QA * 4 * NT == BM * BK && QB * 4 * NT == BN * BK, "tile not divisible by the loaders");
    static_assert(CA * 256 * NW == AS && CB * 256 * NW == BS, "tile not divisible into LDS chunks");
};

// Configurations of the grouped launches (rotations, Gram products, opt_gemm).
// The large tile: 256 x 256 outputs per workgroup of 2 x 4 wavefronts (128 x
// 64 each) with 16-deep slabs, two wavefronts per SIMD. With the fp32
// products on bf16 MFMAs (96 KiB of LDS, one workgroup per CU) each operand
// value that a workgroup loads and splits feeds 256 outputs instead of 128 or
// 256 on a 256 x 128 tile of 4 wavefronts: 7 % less time on the rotation
// phases (the fill's loads and split per MFMA drop by a quarter).
#ifndef MATOPT_LARGE_CFG
#define MATOPT_LARGE_CFG 2, 4, 4, 2, 16
#endif
using SmallCfg = Cfg<2, 2, 2, 2>;
using LargeCfg = Cfg<MATOPT_LARGE_CFG>;
static_assert(SmallCfg::BM == kGemmCfgs[0].bm && SmallCfg::BN == kGemmCfgs[0].bn, "tile size mismatch");
static_assert(LargeCfg::BM == kGemmCfgs[1].bm && LargeCfg::BN == kGemmCfgs[1].bn, "tile size mismatch");
// Configuration of the QR trailing updates (short K, memory-bound C).
using QrCfg = Cfg<2, 2, 2, 2>;
static_assert(QrCfg::BM == kQrTile && QrCfg::BN == kQrTile, "QR tile size mismatch");

// Slot of 16-byte group q in row r of a k-contiguous LDS operand with BK/4
// groups per row: slot q ^ swz(r). For 8 groups, (r + r/8) mod 8; for 4,
// ((r/2) ^ (r/4)) mod 4. Either way any 8 aligned consecutive rows, and the
// rows of one residue among any 16 aligned consecutive rows, fall on distinct
// 4-bank groups for a 16-byte read.
template <int BK>
__device__ __forceinline__ int swz(int r) {
    if constexpr (BK == 32) return (r + (r >> 3)) & 7;
    else return ((r >> 1) ^ (r >> 2)) & 3;
}

typedef __attribute__((address_space(3))) void* lds_ptr;
typedef __attribute__((address_space(1))) const void* gsrc_ptr;

// Fill one slab of an fp32 operand into LDS buffer `buf` with direct loads.
// The operand is stored row-major with leading dimension ld and `rows` x
// `cols` valid elements. KMAJOR: LDS [32][R] from stored rows k0.. (k) and
// columns c0.. (the tile's m or n); otherwise LDS [R][32] swizzled, from
// stored rows c0.. (m or n) and columns k0.. (k). VEC: 16-byte loads (ld,
// cols and the base 4-aligned); otherwise four 4-byte loads per 16 bytes.
template <class C, bool KMAJOR, int R>
__device__ __forceinline__ void dma_slab(float* buf, const float* base, int64_t ld, int rows, int cols,
                                         int c0, int k0, bool vec) {
    constexpr int BK = C::BK, G = BK / 4;       // groups of 4 k values per row
    constexpr int CPW = R * BK / 256 / C::NW;   // chunks per wavefront
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (vec) {
        const int last = cols - 4;
#pragma unroll
        for (int t = 0; t < CPW; ++t) {
            const int c = wave * CPW + t;
            int grow, gcol;
            if (KMAJOR) {
                const int flat = c * 256 + 4 * lane;
                grow = k0 + flat / R;
                gcol = c0 + flat % R;
            } else {
                const int r = (256 / BK) * c + lane / G;
                grow = c0 + r;
                gcol = k0 + 4 * ((lane % G) ^ swz<BK>(r));
            }
            grow = grow < rows ? grow : rows - 1;
            gcol = gcol < last ? gcol : last;
            __builtin_amdgcn_global_load_lds((gsrc_ptr)(base + (int64_t)grow * ld + gcol),
                                             (lds_ptr)(buf + c * 256), 16, 0, 0);
        }
    } else {
#pragma unroll
        for (int t = 0; t < CPW; ++t) {
            const int c = wave * CPW + t;
#pragma unroll
            for (int e4 = 0; e4 < 4; ++e4) {
                const int f = c * 256 + 64 * e4 + lane;   // LDS float this lane writes
                int grow, gcol;
                if (KMAJOR) {
                    grow = k0 + f / R;
                    gcol = c0 + f % R;
                } else {
                    const int r = f / BK, p = f % BK;
                    grow = c0 + r;
                    gcol = k0 + 4 * ((p >> 2) ^ swz<BK>(r)) + (p & 3);
                }
                grow = grow < rows ? grow : rows - 1;
                gcol = gcol < cols ? gcol : cols - 1;
                __builtin_amdgcn_global_load_lds((gsrc_ptr)(base + (int64_t)grow * ld + gcol),
                                                 (lds_ptr)(buf + c * 256 + 64 * e4), 4, 0, 0);
            }
        }
    }
}

// Zero the k values >= K of a slab filled by dma_slab (a partial last slab).
template <class C, bool KMAJOR, int R>
__device__ __forceinline__ void zero_k_tail(float* buf, int k0, int K) {
    constexpr int BK = C::BK;
    const int kv = K - k0;   // valid k values in this slab, 0 < kv < BK
    for (int e = threadIdx.x; e < R * BK; e += C::NT) {
        if (KMAJOR) {
            if (e / R >= kv) buf[e] = 0.f;
        } else {
            const int r = e / BK, kk = e % BK;
            if (kk >= kv) buf[r * BK + 4 * ((kk >> 2) ^ swz<BK>(r)) + (kk & 3)] = 0.f;
        }
    }
}

// Four consecutive elements (row, col..col+3) of a row-major stored matrix,
// as loaded: fp32 values, or the raw bits of bf16 values. They are widened and
// masked only when stored to LDS, after the current slab's MFMAs, so that the
// load latency of slab k+1 overlaps the MFMAs of slab k.
template <bool BF16> struct Raw4 { f32x4 v; };
template <> struct Raw4<true> { u32x2 v; };

// The address is clamped into the valid `rows` x `cols` region so that every
// lane issues a load at a valid address (no divergent branches); the values
// outside are zeroed at the store. With VEC the load is one 16-byte (fp32) or
// 8-byte (bf16) access, which needs ld % 4 == 0, cols % 4 == 0 and an aligned
// base (so a clamped group never leaves the row).
template <bool BF16>
__device__ __forceinline__ Raw4<BF16> load4(const void* base, int64_t ld, int row, int col, int rows,
                                            int cols, bool vec) {
    const int64_t rc = row < rows ? row : rows - 1;
    Raw4<BF16> r;
    if (vec) {
        const int last = (cols - 1) & ~3;
        const int64_t off = rc * ld + (col < last ? col : last);
        if constexpr (BF16) r.v = *gptr((const u32x2*)((const uint16_t*)base + off));
        else                r.v = *gptr((const f32x4*)((const float*)base + off));
    } else {
        if constexpr (BF16) {
            uint32_t h[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int ce = col + e < cols ? col + e : cols - 1;
                h[e] = gptr((const uint16_t*)base)[rc * ld + ce];
            }
            r.v.x = h[0] | (h[1] << 16);
            r.v.y = h[2] | (h[3] << 16);
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int ce = col + e < cols ? col + e : cols - 1;
                r.v[e] = gptr((const float*)base)[rc * ld + ce];
            }
        }
    }
    return r;
}

// Widen to fp32 and zero the elements outside the valid region.
template <bool BF16>
__device__ __forceinline__ f32x4 finish4(const Raw4<BF16>& r, int row, int col, int rows, int cols) {
    f32x4 v;
    if constexpr (BF16) {
        v[0] = __uint_as_float(r.v.x << 16);
        v[1] = __uint_as_float(r.v.x & 0xffff0000u);
        v[2] = __uint_as_float(r.v.y << 16);
        v[3] = __uint_as_float(r.v.y & 0xffff0000u);
    } else {
        v = r.v;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e)
        if (!(row < rows && col + e < cols)) v[e] = 0.f;
    return v;
}

// Element coordinates of the q-th float4 a thread moves in a slab: for an
// operand kept k-major (A stored K x M, B stored K x N) the slab rows are k
// with W/4 float4 per row; otherwise the slab rows are m (or n) with 8 float4
// per row of 32 k values.
template <class C, bool KMAJOR, int W>
__device__ __forceinline__ void slab_pos(int q, int& rr, int& c4) {
    const int f = threadIdx.x + C::NT * q;
    if (KMAJOR) { rr = f / (W / 4); c4 = f % (W / 4); }
    else        { rr = f / (C::BK / 4); c4 = f % (C::BK / 4); }
}

template <class C, bool AT, bool ABF>
__device__ __forceinline__ void load_a(const GemmProb& p, int m0, int k0, Raw4<ABF> (&r)[C::QA]) {
    const bool vec = p.flags & GF_A_VEC;
#pragma unroll
    for (int q = 0; q < C::QA; ++q) {
        int rr, c4;
        slab_pos<C, AT, C::BM>(q, rr, c4);
        if (AT) r[q] = load4<ABF>(p.A, p.lda, k0 + rr, m0 + 4 * c4, p.K, p.M, vec);
        else    r[q] = load4<ABF>(p.A, p.lda, m0 + rr, k0 + 4 * c4, p.M, p.K, vec);
    }
}

template <class C, bool BT, bool BBF>
__device__ __forceinline__ void load_b(const GemmProb& p, int n0, int k0, Raw4<BBF> (&r)[C::QB]) {
    const bool vec = p.flags & GF_B_VEC;
#pragma unroll
    for (int q = 0; q < C::QB; ++q) {
        int rr, c4;
        slab_pos<C, !BT, C::BN>(q, rr, c4);
        if (BT) r[q] = load4<BBF>(p.B, p.ldb, n0 + rr, k0 + 4 * c4, p.N, p.K, vec);
        else    r[q] = load4<BBF>(p.B, p.ldb, k0 + rr, n0 + 4 * c4, p.K, p.N, vec);
    }
}

// UL: A is read as unit lower trapezoidal (ones on the diagonal, zeros above).
template <class C, bool AT, bool ABF, bool UL>
__device__ __forceinline__ void store_a(float* As, const Raw4<ABF> (&r)[C::QA], const GemmProb& p, int m0,
                                        int k0) {
#pragma unroll
    for (int q = 0; q < C::QA; ++q) {
        int rr, c4;
        slab_pos<C, AT, C::BM>(q, rr, c4);
        if (AT) {
            *(f32x4*)&As[rr * C::BM + 4 * c4] = finish4<ABF>(r[q], k0 + rr, m0 + 4 * c4, p.K, p.M);
        } else {
            const int row = m0 + rr, col = k0 + 4 * c4;
            f32x4 v = finish4<ABF>(r[q], row, col, p.M, p.K);
            if (UL) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    if (row < col + e) v[e] = 0.f;
                    else if (row == col + e) v[e] = 1.f;
                }
            }
            *(f32x4*)&As[rr * C::BK + 4 * (c4 ^ swz<C::BK>(rr))] = v;
        }
    }
}

template <class C, bool BT, bool BBF>
__device__ __forceinline__ void store_b(float* Bs, const Raw4<BBF> (&r)[C::QB], const GemmProb& p, int n0,
                                        int k0) {
#pragma unroll
    for (int q = 0; q < C::QB; ++q) {
        int rr, c4;
        slab_pos<C, !BT, C::BN>(q, rr, c4);
        if (BT) *(f32x4*)&Bs[rr * C::BK + 4 * (c4 ^ swz<C::BK>(rr))] = finish4<BBF>(r[q], n0 + rr, k0 + 4 * c4, p.N, p.K);
        else    *(f32x4*)&Bs[rr * C::BN + 4 * c4] = finish4<BBF>(r[q], k0 + rr, n0 + 4 * c4, p.K, p.N);
    }
}

template <class C>
struct Acc {
    f32x16 v[C::TM][C::TN];
    __device__ __forceinline__ void zero() {
#pragma unroll
        for (int i = 0; i < C::TM; ++i)
#pragma unroll
            for (int j = 0; j < C::TN; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) v[i][j][r] = 0.f;
    }
};

// Operand fragments of k group g (8 k values) of a slab: a[i] feeds the
// MFMAs of row block i, b[j] those of column block j (element s: MFMA s).
template <class C, bool AT, bool BT>
__device__ __forceinline__ void read_frags(const float* As, const float* Bs, int g, int wm, int wn, int lane,
                                           f32x4 (&a)[C::TM], f32x4 (&b)[C::TN]) {
    const int h = lane >> 5, l32 = lane & 31;
#pragma unroll
    for (int i = 0; i < C::TM; ++i) {
        const int row = wm * 32 * C::TM + i * 32 + l32;
        if (AT) {
#pragma unroll
            for (int s = 0; s < 4; ++s) a[i][s] = As[(8 * g + 4 * h + s) * C::BM + row];
        } else {
            a[i] = *(const f32x4*)&As[row * C::BK + 4 * ((2 * g + h) ^ swz<C::BK>(row))];
        }
    }
#pragma unroll
    for (int j = 0; j < C::TN; ++j) {
        const int col = wn * 32 * C::TN + j * 32 + l32;
        if (BT) {
            b[j] = *(const f32x4*)&Bs[col * C::BK + 4 * ((2 * g + h) ^ swz<C::BK>(col))];
        } else {
#pragma unroll
            for (int s = 0; s < 4; ++s) b[j][s] = Bs[(8 * g + 4 * h + s) * C::BN + col];
        }
    }
}

// MFMAs s = S0 .. S1-1 of one k group.
template <class C, int S0 = 0, int S1 = 4>
__device__ __forceinline__ void mma_group(const f32x4 (&a)[C::TM], const f32x4 (&b)[C::TN], Acc<C>& acc) {
#pragma unroll
    for (int s = S0; s < S1; ++s)
#pragma unroll
        for (int i = 0; i < C::TM; ++i)
#pragma unroll
            for (int j = 0; j < C::TN; ++j)
                acc.v[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[i][s], b[j][s], acc.v[i][j], 0, 0, 0);
}

template <class C, bool AT, bool BT>
__device__ __forceinline__ void mma_slab(const float* As, const float* Bs, int wm, int wn, int lane,
                                         Acc<C>& acc) {
    const int h = lane >> 5, l32 = lane & 31;
#pragma unroll
    for (int g = 0; g < C::BK / 8; ++g) {
        f32x4 a[C::TM], b[C::TN];
#pragma unroll
        for (int i = 0; i < C::TM; ++i) {
            const int row = wm * 32 * C::TM + i * 32 + l32;
            if (AT) {
#pragma unroll
                for (int s = 0; s < 4; ++s) a[i][s] = As[(8 * g + 4 * h + s) * C::BM + row];
            } else {
                a[i] = *(const f32x4*)&As[row * C::BK + 4 * ((2 * g + h) ^ swz<C::BK>(row))];
            }
        }
#pragma unroll
        for (int j = 0; j < C::TN; ++j) {
            const int col = wn * 32 * C::TN + j * 32 + l32;
            if (BT) {
                b[j] = *(const f32x4*)&Bs[col * C::BK + 4 * ((2 * g + h) ^ swz<C::BK>(col))];
            } else {
#pragma unroll
                for (int s = 0; s < 4; ++s) b[j][s] = Bs[(8 * g + 4 * h + s) * C::BN + col];
            }
        }
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int i = 0; i < C::TM; ++i)
#pragma unroll
                for (int j = 0; j < C::TN; ++j)
                    acc.v[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[i][s], b[j][s], acc.v[i][j], 0, 0, 0);
    }
}

// ---- fp32 products on bf16 MFMAs (X6 mode) ----
//
// An fp32 value x splits into three bf16 values hi = rb(x), mid = rb(x - hi),
// lo = rb(x - hi - mid) (rb: round to nearest even). Both residuals are exact
// in fp32, and the last has at most 8 significant bits, so hi + mid + lo = x
// exactly for finite x. A product a b is then the sum of the nine piece
// products; the six kept here (hi hi, hi mid, mid hi, hi lo, mid mid, lo hi)
// leave out terms below 2^-23 |a b| in all, about one fp32 rounding of the
// product, and every piece product is exact in the fp32 accumulator. So one
// k step of 16 on v_mfma_f32_32x32x16_bf16 (six MFMAs per 32 x 32 block) does
// the work of eight v_mfma_f32_32x32x2_f32 at fp32 accuracy; the matrix
// cores' bf16 rate being 16 times the fp32 one, it takes 6/16 of the time at
// peak.
//
// The operands stay fp32 in LDS (the same layouts and fills as the fp32
// path); a k step takes the fragments of two consecutive groups of 8 k
// values, and lane l's element e (0..7) of a bf16 fragment is the value of k
// 8 (g + e/4) + 4 (l/32) + e%4: the same assignment for both operands, so the
// sum over the step's 16 k values is unchanged.
struct Pieces {
    bf16x8 hi, mid, lo;
};

// Pairs of values: one v_cvt_pk_bf16_f32 per piece and pair, the widening
// back to fp32 a shift or a mask, the residuals plain fp32 subtractions.
__device__ __forceinline__ void split2(float x0, float x1, uint32_t& hi, uint32_t& mid, uint32_t& lo) {
    const f32x2 x = {x0, x1};
    const bf16x2 h = __builtin_convertvector(x, bf16x2);
    const uint32_t hb = __builtin_bit_cast(uint32_t, h);
    const f32x2 r1 = {x0 - __uint_as_float(hb << 16), x1 - __uint_as_float(hb & 0xffff0000u)};
    const bf16x2 m = __builtin_convertvector(r1, bf16x2);
    const uint32_t mb = __builtin_bit_cast(uint32_t, m);
    const f32x2 r2 = {r1[0] - __uint_as_float(mb << 16), r1[1] - __uint_as_float(mb & 0xffff0000u)};
    hi = hb;
    mid = mb;
    lo = __builtin_bit_cast(uint32_t, __builtin_convertvector(r2, bf16x2));
}

__device__ __forceinline__ Pieces split8(const f32x4& x0, const f32x4& x1) {
    uint32_t h[4], m[4], l[4];
    split2(x0[0], x0[1], h[0], m[0], l[0]);
    split2(x0[2], x0[3], h[1], m[1], l[1]);
    split2(x1[0], x1[1], h[2], m[2], l[2]);
    split2(x1[2], x1[3], h[3], m[3], l[3]);
    Pieces p;
    p.hi = __builtin_bit_cast(bf16x8, (u32x4){h[0], h[1], h[2], h[3]});
    p.mid = __builtin_bit_cast(bf16x8, (u32x4){m[0], m[1], m[2], m[3]});
    p.lo = __builtin_bit_cast(bf16x8, (u32x4){l[0], l[1], l[2], l[3]});
    return p;
}

// One k step of 16 for the blocks of A row block i: the six piece products,
// smallest first.
template <class C>
__device__ __forceinline__ void mma6_row(const Pieces& a, const Pieces (&b)[C::TN], f32x16 (&acc)[C::TN]) {
    // piece product by piece product across the row's column blocks, so that
    // consecutive MFMAs go to different accumulators
#pragma unroll
    for (int j = 0; j < C::TN; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a.lo, b[j].hi, acc[j], 0, 0, 0);
#pragma unroll
    for (int j = 0; j < C::TN; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a.mid, b[j].mid, acc[j], 0, 0, 0);
#pragma unroll
    for (int j = 0; j < C::TN; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a.hi, b[j].lo, acc[j], 0, 0, 0);
#pragma unroll
    for (int j = 0; j < C::TN; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a.mid, b[j].hi, acc[j], 0, 0, 0);
#pragma unroll
    for (int j = 0; j < C::TN; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a.hi, b[j].mid, acc[j], 0, 0, 0);
#pragma unroll
    for (int j = 0; j < C::TN; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a.hi, b[j].hi, acc[j], 0, 0, 0);
}

// Accumulator register r of lane l holds row 8*(r/4) + 4*(l/32) + r%4,
// column l%32 of its 32x32 block: 32 lanes store 128 contiguous bytes.
// With beta != 0 the old values of one row of blocks are all loaded before
// any of them is stored (a store to C could otherwise alias a later load as
// far as the compiler can tell, serialising them).
template <class C>
__device__ __forceinline__ void epilogue(const GemmProb& p, int m0, int n0, int wm, int wn, int lane,
                                         const Acc<C>& acc, float alpha, float beta) {
    const int h = lane >> 5, l32 = lane & 31;
#pragma unroll
    for (int i = 0; i < C::TM; ++i) {
        float cold[C::TN][16];
        if (beta != 0.f) {
#pragma unroll
            for (int j = 0; j < C::TN; ++j) {
                const int col = n0 + wn * 32 * C::TN + j * 32 + l32;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int row = m0 + wm * 32 * C::TM + i * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
                    cold[j][r] = (row < p.M && col < p.N) ? gptr(p.C)[(int64_t)row * p.ldc + col] : 0.f;
                }
            }
        }
#pragma unroll
        for (int j = 0; j < C::TN; ++j) {
            const int col = n0 + wn * 32 * C::TN + j * 32 + l32;
            if (col >= p.N) continue;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = m0 + wm * 32 * C::TM + i * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
                if (row < p.M) {
                    float val = alpha * acc.v[i][j][r];
                    if (beta != 0.f) val += beta * cold[j][r];
                    gptr(p.C)[(int64_t)row * p.ldc + col] = val;
                }
            }
        }
    }
}

// The same stores one 32 x 32 block at a time (old values of the block
// loaded first), for tiles whose main loop leaves fewer registers free.
template <class C>
__device__ __forceinline__ void epilogue_blocks(const GemmProb& p, int m0, int n0, int wm, int wn, int lane,
                                                const Acc<C>& acc, float alpha, float beta) {
    const int h = lane >> 5, l32 = lane & 31;
#pragma unroll
    for (int i = 0; i < C::TM; ++i) {
#pragma unroll
        for (int j = 0; j < C::TN; ++j) {
            const int col = n0 + wn * 32 * C::TN + j * 32 + l32;
            const int row0 = m0 + wm * 32 * C::TM + i * 32 + 4 * h;
            float cold[16];
            if (beta != 0.f) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int row = row0 + 8 * (r >> 2) + (r & 3);
                    cold[r] = (row < p.M && col < p.N) ? gptr(p.C)[(int64_t)row * p.ldc + col] : 0.f;
                }
            }
            if (col >= p.N) continue;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = row0 + 8 * (r >> 2) + (r & 3);
                if (row < p.M) {
                    float val = alpha * acc.v[i][j][r];
                    if (beta != 0.f) val += beta * cold[r];
                    gptr(p.C)[(int64_t)row * p.ldc + col] = val;
                }
            }
        }
    }
}

template <class C, bool AT, bool BT, bool ABF, bool BBF, bool X6>
__device__ __forceinline__ void gemm_tile(const GemmProb& p, int tm, int tn, float alpha_scale,
                                          float* smem) {
    constexpr int AS = C::AS, BS = C::BS;
    // buffer b of A at smem + b*AS, of B at smem + 2*AS + b*BS; selected
    // arithmetically so that the slab body is one straight-line block (a
    // branch between two copies makes the compiler move every accumulator
    // between register files at the join)
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave % C::WM, wn = wave / C::WM;
    const int m0 = tm * C::BM, n0 = tn * C::BN;
    const bool avec = p.flags & GF_A_VEC, bvec = p.flags & GF_B_VEC;

    // direct fills of the fp32 operands, and the zeroing of k >= K after a
    // partial slab has landed
    auto fill = [&](int b, int k0) {
        if constexpr (!ABF)
            dma_slab<C, AT, C::BM>(smem + b * AS, (const float*)p.A, p.lda, AT ? p.K : p.M, AT ? p.M : p.K,
                                   m0, k0, avec);
        if constexpr (!BBF)
            dma_slab<C, !BT, C::BN>(smem + 2 * AS + b * BS, (const float*)p.B, p.ldb, BT ? p.N : p.K,
                                    BT ? p.K : p.N, n0, k0, bvec);
    };
    auto tail = [&](int b, int k0) {
        if constexpr (!ABF) zero_k_tail<C, AT, C::BM>(smem + b * AS, k0, p.K);
        if constexpr (!BBF) zero_k_tail<C, !BT, C::BN>(smem + 2 * AS + b * BS, k0, p.K);
    };

    Acc<C> acc;
    acc.zero();
    constexpr int BK = C::BK, NG = BK / 8;   // k groups of 8 per slab
    const int nk = (p.K + BK - 1) / BK;
    if (nk == 0) {
        epilogue<C>(p, m0, n0, wm, wn, lane, acc, p.alpha * alpha_scale, p.beta);
        return;
    }
    Raw4<ABF> ra[ABF ? C::QA : 1];
    Raw4<BBF> rb[BBF ? C::QB : 1];
    fill(0, 0);
    if constexpr (ABF) { load_a<C, AT, ABF>(p, m0, 0, ra); store_a<C, AT, ABF, false>(smem, ra, p, m0, 0); }
    if constexpr (BBF) { load_b<C, BT, BBF>(p, n0, 0, rb); store_b<C, BT, BBF>(smem + 2 * AS, rb, p, n0, 0); }
    __syncthreads();
    if (p.K < BK) {
        tail(0, 0);
        __syncthreads();
    }

    if constexpr (X6) {
        // fp32 products on bf16 MFMAs, one k step of 16 (two groups of 8) at
        // a time. B's fragments of the step are split first; then row block
        // by row block, A's fragments of block i + 1 are read while block i
        // is split and its MFMAs issue, so only one block of A is live. The
        // slab barrier sits before the last row block's MFMAs, and the next
        // slab's B and first A fragments are read behind it, so their latency
        // overlaps those MFMAs.
        static_assert(NG % 2 == 0, "k steps of two groups");
        const int h = lane >> 5, l32 = lane & 31;
        auto frag_a = [&](const float* As, int g, int i) {
            const int row = wm * 32 * C::TM + i * 32 + l32;
            f32x4 a;
            if (AT) {
#pragma unroll
                for (int e = 0; e < 4; ++e) a[e] = As[(8 * g + 4 * h + e) * C::BM + row];
            } else {
                a = *(const f32x4*)&As[row * C::BK + 4 * ((2 * g + h) ^ swz<C::BK>(row))];
            }
            return a;
        };
        auto frag_b = [&](const float* Bs, int g, int j) {
            const int col = wn * 32 * C::TN + j * 32 + l32;
            f32x4 b;
            if (BT) {
                b = *(const f32x4*)&Bs[col * C::BK + 4 * ((2 * g + h) ^ swz<C::BK>(col))];
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) b[e] = Bs[(8 * g + 4 * h + e) * C::BN + col];
            }
            return b;
        };
        // fragments of the current k step: B (both groups) and A's row block 0
        f32x4 b0[C::TN], b1[C::TN], a0, a1;
#pragma unroll
        for (int j = 0; j < C::TN; ++j) {
            b0[j] = frag_b(smem + 2 * AS, 0, j);
            b1[j] = frag_b(smem + 2 * AS, 1, j);
        }
        a0 = frag_a(smem, 0, 0);
        a1 = frag_a(smem, 1, 0);
        for (int kt = 0; kt < nk; ++kt) {
            const int cur = kt & 1;
            const int k1 = (kt + 1) * BK;
            const float* As = smem + cur * AS;
            const float* Bs = smem + 2 * AS + cur * BS;
            const float* An = smem + (cur ^ 1) * AS;
            const float* Bn = smem + 2 * AS + (cur ^ 1) * BS;
            fill(cur ^ 1, k1);
            if constexpr (ABF) load_a<C, AT, ABF>(p, m0, k1, ra);
            if constexpr (BBF) load_b<C, BT, BBF>(p, n0, k1, rb);
#pragma unroll
            for (int st = 0; st < NG / 2; ++st) {
                Pieces pb[C::TN];
#pragma unroll
                for (int j = 0; j < C::TN; ++j) pb[j] = split8(b0[j], b1[j]);
#pragma unroll
                for (int i = 0; i < C::TM; ++i) {
                    const Pieces pa = split8(a0, a1);
                    if (i + 1 < C::TM) {
                        a0 = frag_a(As, 2 * st, i + 1);
                        a1 = frag_a(As, 2 * st + 1, i + 1);
                    } else if (st + 1 < NG / 2) {
                        // the next k step of the same slab
#pragma unroll
                        for (int j = 0; j < C::TN; ++j) {
                            b0[j] = frag_b(Bs, 2 * st + 2, j);
                            b1[j] = frag_b(Bs, 2 * st + 3, j);
                        }
                        a0 = frag_a(As, 2 * st + 2, 0);
                        a1 = frag_a(As, 2 * st + 3, 0);
                    } else {
                        // every fragment of this slab is in registers: the slab
                        // barrier goes before the last row block's MFMAs, and
                        // the next slab's first fragments are read behind it
                        // (past the last slab: values unused)
                        if constexpr (ABF) store_a<C, AT, ABF, false>(smem + (cur ^ 1) * AS, ra, p, m0, k1);
                        if constexpr (BBF) store_b<C, BT, BBF>(smem + 2 * AS + (cur ^ 1) * BS, rb, p, n0, k1);
                        __syncthreads();
                        if (k1 < p.K && k1 + BK > p.K) {
                            tail(cur ^ 1, k1);
                            __syncthreads();
                        }
#pragma unroll
                        for (int j = 0; j < C::TN; ++j) {
                            b0[j] = frag_b(Bn, 0, j);
                            b1[j] = frag_b(Bn, 1, j);
                        }
                        a0 = frag_a(An, 0, 0);
                        a1 = frag_a(An, 1, 0);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                    mma6_row<C>(pa, pb, acc.v[i]);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        }
        epilogue_blocks<C>(p, m0, n0, wm, wn, lane, acc, p.alpha * alpha_scale, p.beta);
        return;
    }

    // Software pipeline over the four k groups of a slab: the fragments of
    // group g+1 are read after the first MFMAs of group g have been issued,
    // so every wait for a fragment finds it read a group earlier. The slab's
    // closing barrier sits before the MFMAs of its last group, and the reads
    // of the next slab's first group follow right after it. The fill of slab
    // kt+1 is issued unconditionally: past the last slab it reads clamped,
    // valid addresses into the idle buffer, which keeps the slab body one
    // basic block.
    f32x4 fa[2][C::TM], fb[2][C::TN];
    read_frags<C, AT, BT>(smem, smem + 2 * AS, 0, wm, wn, lane, fa[0], fb[0]);
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        const int k1 = (kt + 1) * BK;
        const float* As = smem + cur * AS;
        const float* Bs = smem + 2 * AS + cur * BS;
        fill(cur ^ 1, k1);
        if constexpr (ABF) load_a<C, AT, ABF>(p, m0, k1, ra);
        if constexpr (BBF) load_b<C, BT, BBF>(p, n0, k1, rb);
#pragma unroll
        for (int g = 0; g < NG - 1; ++g) {
            mma_group<C, 0, 1>(fa[g & 1], fb[g & 1], acc);
            __builtin_amdgcn_sched_barrier(0);
            read_frags<C, AT, BT>(As, Bs, g + 1, wm, wn, lane, fa[(g + 1) & 1], fb[(g + 1) & 1]);
            __builtin_amdgcn_sched_barrier(0);
            mma_group<C, 1, 4>(fa[g & 1], fb[g & 1], acc);
            __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (ABF) store_a<C, AT, ABF, false>(smem + (cur ^ 1) * AS, ra, p, m0, k1);
        if constexpr (BBF) store_b<C, BT, BBF>(smem + 2 * AS + (cur ^ 1) * BS, rb, p, n0, k1);
        __syncthreads();
        if (k1 < p.K && k1 + BK > p.K) {
            tail(cur ^ 1, k1);
            __syncthreads();
        }
        // the last group, with the next slab's first group read behind its
        // first MFMAs (past the last slab: values unused)
        static_assert(NG % 2 == 0, "the last group's fragments are in slot 1");
        mma_group<C, 0, 1>(fa[1], fb[1], acc);
        __builtin_amdgcn_sched_barrier(0);
        read_frags<C, AT, BT>(smem + (cur ^ 1) * AS, smem + 2 * AS + (cur ^ 1) * BS, 0, wm, wn, lane, fa[0], fb[0]);
        __builtin_amdgcn_sched_barrier(0);
        mma_group<C, 1, 4>(fa[1], fb[1], acc);
        __builtin_amdgcn_sched_barrier(0);
    }
    epilogue<C>(p, m0, n0, wm, wn, lane, acc, p.alpha * alpha_scale, p.beta);
}

// ---- fp32 products on bf16 MFMAs, each operand value split once ----
//
// The X6 products of the grouped launches. Each workgroup loads a 16-deep k
// slab of both operands from global memory into registers, splits every
// value once into its three bf16 pieces (split2 above) and writes the pieces
// to LDS as three planes; the wavefronts then read ready bf16 fragments, so
// no value is split twice (a wavefront that split its own fragments would
// split each A and B value once per wavefront that reads it: twice in a
// 2 x 2 arrangement). LDS holds two slabs; the pieces of slab k + 1 are
// written while slab k's MFMAs run, and slab k + 2 is loaded into registers
// behind them: one barrier per slab.
//
// LDS layout: per operand and piece a plane of R rows (the tile's m or n)
// by 16 k values in bf16, 32 bytes per row. MFMA lane l takes 8 bf16 of
// row l % 32 at k = 8 (l / 32) .. +7 (one ds_read_b128, the same k order for
// A and B); half h of row r sits at byte 32 r + 16 (h ^ ((r / 8) % 2)), which
// puts the sixteen rows that one phase of a read touches on distinct 16-byte
// bank groups.
//
// Fills: an operand whose k index is contiguous in memory is loaded 16 bytes
// (four k values) per lane, four lanes per row; one whose k index is the
// memory row (k-major) is loaded four k rows at a time, one element per lane,
// the lanes along the contiguous index. Rows past the operand, and k past K,
// are loaded from clamped addresses and zeroed before the split. A bf16
// operand (A or B, not both) is exact in its high piece: its plane is the
// loaded value, and the three products with its zero pieces are skipped; with
// k contiguous it is loaded four k values (8 bytes) per lane.

// The X6 products split each value once, at the fill (gemm_x6_kernel);
// MATOPT_X6_REGISTER_SPLIT (kX6SplitAtFill false) selects the in-register
// split of gemm_grouped_kernel's X6 path instead.

template <class C, bool ABF, bool BBF>
struct X6Lds {
    static constexpr int PA = C::BM * 32;   // bytes of one A piece plane
    static constexpr int PB = C::BN * 32;
    static constexpr int NPA = ABF ? 1 : 3;
    static constexpr int NPB = BBF ? 1 : 3;
    static constexpr int BUF = NPA * PA + NPB * PB;
    static constexpr int BYTES = 2 * BUF;
};

__device__ __forceinline__ int x6_off(int r, int half) { return r * 32 + 16 * (half ^ ((r >> 3) & 1)); }

// One operand's slab in registers: R rows of 16 k values as halves of eight
// k values, H halves per thread. A thread's half of a row is one 16-byte
// write per piece plane (the half's slot in LDS, x6_off(r, h)). An operand
// whose k index is the memory row (k-major) gives consecutive lanes
// consecutive rows, so that each of its eight loads is coalesced across the
// wavefront; the 16-byte writes then go to rows 32 bytes apart, which with
// the half swizzle cover all banks once per 16 lanes (8-byte writes at that
// stride had four-way bank conflicts). A k-contiguous operand gives each row
// to two consecutive lanes (16 or 32 contiguous bytes per lane).
//
// Addresses: at the start of a tile each half's byte offset from the
// operand's slab-0 origin is computed once (its row clamped into the
// operand), 32-bit since an operand of the step is at most 2^30 bytes (a
// larger one takes the clamped path throughout). A slab whose 16 k values
// all lie inside K then loads from the slab's origin, a uniform address,
// plus those offsets; only a last, partial slab recomputes clamped
// addresses.
template <int R, bool KMAJ, bool BF, int NT>
struct X6Fill {
    static constexpr int H = R * 2 / NT;
    static constexpr int ES = BF ? 2 : 4;   // element bytes
    static_assert(H * NT == R * 2, "tile rows not divisible among the threads");
    float v[H][8];
    uint32_t off[H];

    // half i of this thread: row r (0..R-1) of the tile, half o (0, 1) of the slab
    __device__ __forceinline__ static void pos(int i, int& r, int& o) {
        const int f = (int)threadIdx.x + NT * i;
        if (KMAJ) { r = f % R; o = f / R; }
        else      { r = f >> 1; o = f & 1; }
    }

    __device__ __forceinline__ void init(int64_t ld, int r0, int rows_v) {
#pragma unroll
        for (int i = 0; i < H; ++i) {
            int r, o;
            pos(i, r, o);
            const int row = r0 + r;
            const int rc = row < rows_v ? row : rows_v - 1;
            off[i] = KMAJ ? (uint32_t)(((int64_t)(8 * o) * ld + rc) * ES) : (uint32_t)(((int64_t)rc * ld + 8 * o) * ES);
        }
    }

    // A slab inside K: origin = the operand's element (k0, row 0) (k-major)
    // or (row 0, k0); `vec`: 16-byte (fp32) / 8-byte (bf16) aligned groups
    // of four k values.
    __device__ __forceinline__ void load_inner(const char* origin, int64_t ld, bool vec) {
        const gmem<const char> o = gptr(origin);
#pragma unroll
        for (int i = 0; i < H; ++i) {
            if (KMAJ) {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const gmem<const char> pe = o + (int64_t)e * ld * ES;
                    if constexpr (BF)
                        v[i][e] = __uint_as_float((uint32_t)*(const gmem<const uint16_t>)(pe + off[i]) << 16);
                    else
                        v[i][e] = *(const gmem<const float>)(pe + off[i]);
                }
            } else if (vec) {
#pragma unroll
                for (int g = 0; g < 2; ++g) {
                    if constexpr (BF) {
                        const u32x2 x = *(const gmem<const u32x2>)(o + off[i] + 8 * g);
                        v[i][4 * g + 0] = __uint_as_float(x[0] << 16);
                        v[i][4 * g + 1] = __uint_as_float(x[0] & 0xffff0000u);
                        v[i][4 * g + 2] = __uint_as_float(x[1] << 16);
                        v[i][4 * g + 3] = __uint_as_float(x[1] & 0xffff0000u);
                    } else {
                        const f32x4 x = *(const gmem<const f32x4>)(o + off[i] + 16 * g);
#pragma unroll
                        for (int e = 0; e < 4; ++e) v[i][4 * g + e] = x[e];
                    }
                }
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    if constexpr (BF)
                        v[i][e] = __uint_as_float((uint32_t)*(const gmem<const uint16_t>)(o + off[i] + e * ES) << 16);
                    else
                        v[i][e] = *(const gmem<const float>)(o + off[i] + e * ES);
                }
            }
        }
    }

    // Any slab, addresses clamped into the operand. base: the operand;
    // rows_v: valid rows (m or n), K; ld: leading dimension.
    __device__ __forceinline__ void load_clamped(const void* base, int64_t ld, int r0, int rows_v, int k0, int K,
                                                 bool vec) {
#pragma unroll
        for (int i = 0; i < H; ++i) {
            int r, o;
            pos(i, r, o);
            const int row = r0 + r;
            const int rc = row < rows_v ? row : rows_v - 1;
#pragma unroll
            for (int g = 0; g < 2; ++g) {
                const int kq = k0 + 8 * o + 4 * g;   // first k of this group of four
                if (KMAJ) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int ke = kq + e < K ? kq + e : K - 1;
                        if constexpr (BF)
                            v[i][4 * g + e] = __uint_as_float((uint32_t)gptr((const uint16_t*)base)[(int64_t)ke * ld + rc] << 16);
                        else
                            v[i][4 * g + e] = gptr((const float*)base)[(int64_t)ke * ld + rc];
                    }
                } else if (vec) {
                    const int last = (K - 1) & ~3;
                    const int kc = kq < last ? kq : last;
                    if constexpr (BF) {
                        const u32x2 x = *gptr((const u32x2*)((const uint16_t*)base + (int64_t)rc * ld + kc));
                        v[i][4 * g + 0] = __uint_as_float(x[0] << 16);
                        v[i][4 * g + 1] = __uint_as_float(x[0] & 0xffff0000u);
                        v[i][4 * g + 2] = __uint_as_float(x[1] << 16);
                        v[i][4 * g + 3] = __uint_as_float(x[1] & 0xffff0000u);
                    } else {
                        const f32x4 x = *gptr((const f32x4*)((const float*)base + (int64_t)rc * ld + kc));
#pragma unroll
                        for (int e = 0; e < 4; ++e) v[i][4 * g + e] = x[e];
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int ke = kq + e < K ? kq + e : K - 1;
                        if constexpr (BF)
                            v[i][4 * g + e] = __uint_as_float((uint32_t)gptr((const uint16_t*)base)[(int64_t)rc * ld + ke] << 16);
                        else
                            v[i][4 * g + e] = gptr((const float*)base)[(int64_t)rc * ld + ke];
                    }
                }
            }
        }
    }

    // Split and write the planes (plane p at `lds` + p * plane_bytes); with
    // `mask`, first zero what lies outside the operand (rows past rows_v, k
    // past K), which the clamped loads read as copies of the last row or k.
    __device__ __forceinline__ void put(char* lds, int plane_bytes, bool mask, int r0, int rows_v, int k0,
                                        int K) const {
#pragma unroll
        for (int i = 0; i < H; ++i) {
            int r, o;
            pos(i, r, o);
            float x[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] = v[i][e];
            if (mask) {
                const bool row_ok = r0 + r < rows_v;
#pragma unroll
                for (int e = 0; e < 8; ++e) x[e] = (row_ok && k0 + 8 * o + e < K) ? x[e] : 0.f;
            }
            const int off = x6_off(r, o);
            if constexpr (BF) {
                // exact bf16 values: the high halves of the widened words
                u32x4 w;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    w[e] = (__float_as_uint(x[2 * e]) >> 16) | (__float_as_uint(x[2 * e + 1]) & 0xffff0000u);
                *(u32x4*)(lds + off) = w;
            } else {
                u32x4 hi, mid, lo;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    uint32_t h, m, l;
                    split2(x[2 * e], x[2 * e + 1], h, m, l);
                    hi[e] = h;
                    mid[e] = m;
                    lo[e] = l;
                }
                *(u32x4*)(lds + off) = hi;
                *(u32x4*)(lds + plane_bytes + off) = mid;
                *(u32x4*)(lds + 2 * plane_bytes + off) = lo;
            }
        }
    }
};

// Slabs loaded into registers ahead of their LDS write: 1 (slab k + 2 is
// loaded while slab k's MFMAs run) or 2 (slabs k + 2 and k + 3 in flight, two
// register sets used alternately).
#ifndef MATOPT_X6_PREFETCH
#define MATOPT_X6_PREFETCH 1
#endif
static_assert(MATOPT_X6_PREFETCH == 1 || MATOPT_X6_PREFETCH == 2, "one or two slabs in registers");

template <class C, bool AT, bool BT, bool ABF, bool BBF>
__device__ __forceinline__ void gemm_tile_x6(const GemmProb& p, int tm, int tn, float alpha_scale, char* smem) {
    using L = X6Lds<C, ABF, BBF>;
    constexpr int TM = C::TM, TN = C::TN, NPA = L::NPA, NPB = L::NPB;
    static_assert(!(ABF && BBF), "a product of two bf16 operands needs no pieces");
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave % C::WM, wn = wave / C::WM;
    const int m0 = tm * C::BM, n0 = tn * C::BN;
    const int h = lane >> 5, l32 = lane & 31;
    const bool avec = p.flags & GF_A_VEC, bvec = p.flags & GF_B_VEC;

    Acc<C> acc;
    acc.zero();
    const int nk = (p.K + 15) / 16;
    if (nk == 0) {
        epilogue_blocks<C>(p, m0, n0, wm, wn, lane, acc, p.alpha * alpha_scale, p.beta);
        return;
    }
    // A: M x K (k contiguous) or stored K x M (k-major); B: stored K x N
    // (k-major) or N x K (k contiguous)
    using FA = X6Fill<C::BM, AT, ABF, C::NT>;
    using FB = X6Fill<C::BN, !BT, BBF, C::NT>;
    FA fa0, fa1;
    FB fb0, fb1;
    // the fast path: both operands' bytes addressable with 32-bit offsets
    const int64_t a_span = (int64_t)(AT ? p.K : p.M) * p.lda * FA::ES;
    const int64_t b_span = (int64_t)(BT ? p.N : p.K) * p.ldb * FB::ES;
    const bool offs = a_span < (int64_t(1) << 32) && b_span < (int64_t(1) << 32);
    if (offs) {
        fa0.init(p.lda, m0, p.M);
        fb0.init(p.ldb, n0, p.N);
        if constexpr (MATOPT_X6_PREFETCH == 2) {
#pragma unroll
            for (int i = 0; i < FA::H; ++i) fa1.off[i] = fa0.off[i];
#pragma unroll
            for (int i = 0; i < FB::H; ++i) fb1.off[i] = fb0.off[i];
        }
    }
    const bool rows_partial = m0 + C::BM > p.M || n0 + C::BN > p.N;
    auto load = [&](FA& fa, FB& fb, int k0) {
        if (offs && k0 + 16 <= p.K) {
            fa.load_inner((const char*)p.A + (int64_t)k0 * (AT ? p.lda : 1) * FA::ES, p.lda, avec);
            fb.load_inner((const char*)p.B + (int64_t)k0 * (BT ? 1 : p.ldb) * FB::ES, p.ldb, bvec);
        } else {
            fa.load_clamped(p.A, p.lda, m0, p.M, k0, p.K, avec);
            fb.load_clamped(p.B, p.ldb, n0, p.N, k0, p.K, bvec);
        }
    };
    auto put = [&](const FA& fa, const FB& fb, char* buf, int k0) {
        // interior slabs skip the zeroing, except with a bf16 operand, where
        // the branch made the compiler keep more values live and spill
        const bool mask = ABF || BBF || rows_partial || k0 + 16 > p.K;
        fa.put(buf, L::PA, mask, m0, p.M, k0, p.K);
        fb.put(buf + NPA * L::PA, L::PB, mask, n0, p.N, k0, p.K);
    };
    // slabs past K are loaded from clamped addresses and zeroed at their put
    load(fa0, fb0, 0);
    put(fa0, fb0, smem, 0);
    load(fa0, fb0, 16);
    if constexpr (MATOPT_X6_PREFETCH == 2) load(fa1, fb1, 32);
    __syncthreads();

    // one slab: its MFMAs from LDS buffer kt % 2; after one of its row
    // blocks, slab kt + 1 from registers (fa, fb) into the other buffer and
    // the load of slab kt + 1 + MATOPT_X6_PREFETCH into the same registers.
    // With both operands split, the two wavefronts that share a SIMD (w and
    // w + 4 of 8) split and write the next slab at different row blocks, so
    // that one's vector work meets the other's MFMAs instead of both leaving
    // the matrix unit idle at once (they start each slab together, after its
    // barrier). With one bf16 operand the split is half as long, and the
    // common row block is faster.
    const bool put_late = !ABF && !BBF && C::NT > 256 && (__builtin_amdgcn_readfirstlane(wave) >> 2) % 2 == 1;
    auto slab = [&](int kt, FA& fa, FB& fb) {
        const char* cur = smem + (kt & 1) * L::BUF;
        char* nxt = smem + ((kt + 1) & 1) * L::BUF;
        const char* Bp = cur + NPA * L::PA;
        bf16x8 b[TN][NPB];
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int off = x6_off(wn * 32 * TN + j * 32 + l32, h);
#pragma unroll
            for (int q = 0; q < NPB; ++q) b[j][q] = *(const bf16x8*)(Bp + q * L::PB + off);
        }
        bf16x8 a[NPA];
        {
            const int off = x6_off(wm * 32 * TM + l32, h);
#pragma unroll
            for (int q = 0; q < NPA; ++q) a[q] = *(const bf16x8*)(cur + q * L::PA + off);
        }
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            bf16x8 an[NPA];
            if (i + 1 < TM) {
                const int off = x6_off(wm * 32 * TM + (i + 1) * 32 + l32, h);
#pragma unroll
                for (int q = 0; q < NPA; ++q) an[q] = *(const bf16x8*)(cur + q * L::PA + off);
            }
            __builtin_amdgcn_sched_barrier(0);
            // smallest piece products first; consecutive MFMAs go to
            // different accumulators
            if constexpr (BBF) {
#pragma unroll
                for (int j = 0; j < TN; ++j) acc.v[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[2], b[j][0], acc.v[i][j], 0, 0, 0);
#pragma unroll
                for (int j = 0; j < TN; ++j) acc.v[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[1], b[j][0], acc.v[i][j], 0, 0, 0);
#pragma unroll
                for (int j = 0; j < TN; ++j) acc.v[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[0], b[j][0], acc.v[i][j], 0, 0, 0);
            } else if constexpr (ABF) {
#pragma unroll
                for (int j = 0; j < TN; ++j) acc.v[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[0], b[j][2], acc.v[i][j], 0, 0, 0);
#pragma unroll
                for (int j = 0; j < TN; ++j) acc.v[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[0], b[j][1], acc.v[i][j], 0, 0, 0);
#pragma unroll
                for (int j = 0; j < TN; ++j) acc.v[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[0], b[j][0], acc.v[i][j], 0, 0, 0);
            } else {
#pragma unroll
                for (int j = 0; j < TN; ++j) acc.v[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[2], b[j][0], acc.v[i][j], 0, 0, 0);
#pragma unroll
                for (int j = 0; j < TN; ++j) acc.v[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[1], b[j][1], acc.v[i][j], 0, 0, 0);
#pragma unroll
                for (int j = 0; j < TN; ++j) acc.v[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[0], b[j][2], acc.v[i][j], 0, 0, 0);
#pragma unroll
                for (int j = 0; j < TN; ++j) acc.v[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[1], b[j][0], acc.v[i][j], 0, 0, 0);
#pragma unroll
                for (int j = 0; j < TN; ++j) acc.v[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[0], b[j][1], acc.v[i][j], 0, 0, 0);
#pragma unroll
                for (int j = 0; j < TN; ++j) acc.v[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[0], b[j][0], acc.v[i][j], 0, 0, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
            if (put_late ? i == TM / 2 : i == 0) {
                // the next slab's pieces into the other buffer (read by every
                // wavefront before the previous barrier), then the next load
                put(fa, fb, nxt, (kt + 1) * 16);
                load(fa, fb, (kt + 1 + MATOPT_X6_PREFETCH) * 16);
            }
            if (i + 1 < TM) {
#pragma unroll
                for (int q = 0; q < NPA; ++q) a[q] = an[q];
            }
        }
        __syncthreads();
    };
    if constexpr (MATOPT_X6_PREFETCH == 2) {
        for (int kt = 0; kt < nk; kt += 2) {
            slab(kt, fa0, fb0);
            if (kt + 1 < nk) slab(kt + 1, fa1, fb1);
        }
    } else {
        for (int kt = 0; kt < nk; ++kt) slab(kt, fa0, fb0);
    }
    epilogue_blocks<C>(p, m0, n0, wm, wn, lane, acc, p.alpha * alpha_scale, p.beta);
}

// C += alpha A B for K <= 2 slabs (the QR in-block updates, K = the panel
// width): both K slabs go to the two LDS buffers at once, then the old C
// fragment is requested so that its latency overlaps the MFMAs; the operand
// staging registers are dead by then. A is not transposed and read as unit
// lower trapezoidal (the stored reflectors), B is stored K x N, both fp32.
static_assert(kQrPB <= 2 * QrCfg::BK, "the QR update tile holds the whole panel width in two LDS slabs");

__device__ __forceinline__ void qr_update_tile(const GemmProb& p, int tm, int tn, float* smem) {
    using C = QrCfg;
    constexpr int BK = C::BK;
    constexpr int AS = C::AS, BS = C::BS;
    float* As0 = smem;
    float* As1 = smem + AS;
    float* Bs0 = smem + 2 * AS;
    float* Bs1 = smem + 2 * AS + BS;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave % C::WM, wn = wave / C::WM;
    const int m0 = tm * C::BM, n0 = tn * C::BN;
    const int nk = (p.K + BK - 1) / BK;
    {
        Raw4<false> ra[C::QA], rb[C::QB];
        load_a<C, false, false>(p, m0, 0, ra);
        load_b<C, false, false>(p, n0, 0, rb);
        store_a<C, false, false, true>(As0, ra, p, m0, 0);
        store_b<C, false, false>(Bs0, rb, p, n0, 0);
        if (nk > 1) {
            load_a<C, false, false>(p, m0, BK, ra);
            load_b<C, false, false>(p, n0, BK, rb);
            store_a<C, false, false, true>(As1, ra, p, m0, BK);
            store_b<C, false, false>(Bs1, rb, p, n0, BK);
        }
    }
    __syncthreads();
    const int h = lane >> 5, l32 = lane & 31;
    float cold[C::TM][C::TN][16];
#pragma unroll
    for (int i = 0; i < C::TM; ++i)
#pragma unroll
        for (int j = 0; j < C::TN; ++j) {
            const int col = n0 + wn * 32 * C::TN + j * 32 + l32;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = m0 + wm * 32 * C::TM + i * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
                cold[i][j][r] = (row < p.M && col < p.N) ? gptr(p.C)[(int64_t)row * p.ldc + col] : 0.f;
            }
        }
    Acc<C> acc;
    acc.zero();
    mma_slab<C, false, false>(As0, Bs0, wm, wn, lane, acc);
    if (nk > 1) mma_slab<C, false, false>(As1, Bs1, wm, wn, lane, acc);
#pragma unroll
    for (int i = 0; i < C::TM; ++i)
#pragma unroll
        for (int j = 0; j < C::TN; ++j) {
            const int col = n0 + wn * 32 * C::TN + j * 32 + l32;
            if (col >= p.N) continue;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = m0 + wm * 32 * C::TM + i * 32 + 8 * (r >> 2) + 4 * h + (r & 3);
                if (row < p.M) gptr(p.C)[(int64_t)row * p.ldc + col] = p.alpha * acc.v[i][j][r] + p.beta * cold[i][j][r];
            }
        }
}

// Tile -> (row, column) of tiles, grouped by GROUP_M tile rows for L2 reuse.
__device__ __forceinline__ void raster(int t, int tiles_m, int tiles_n, int& tm, int& tn) {
    const int per_group = GROUP_M * tiles_n;
    const int gidx = t / per_group;
    const int first = gidx * GROUP_M;
    const int gsz = min(tiles_m - first, GROUP_M);
    const int r = t - gidx * per_group;
    tm = first + r % gsz;
    tn = r / gsz;
}

// Workgroup id -> logical tile: within each full window of XCD*XCD_RUN ids,
// the ids the dispatcher sends to one XCD get XCD_RUN consecutive tiles.
__device__ __forceinline__ int xcd_remap(int bid, int total) {
    const int win = XCD * XCD_RUN;
    const int w0 = (bid / win) * win;
    if (w0 + win > total) return bid;
    const int r = bid - w0;
    return w0 + (r % XCD) * XCD_RUN + r / XCD;
}

// A launch's problems: a device table (nprob > 0) or one problem passed by
// value (nprob == 0, used by opt_gemm).
struct GemmArgs {
    const GemmProb* probs;
    const int32_t* tile_begin;
    int nprob;
    int total_tiles;
    float alpha_scale;
    GemmProb single;
};

template <class C, bool AT, bool BT, bool ABF, bool BBF, bool X6>
__global__ __launch_bounds__(C::NT) __attribute__((amdgpu_waves_per_eu(2))) void gemm_grouped_kernel(GemmArgs args) {
    __shared__ __attribute__((aligned(16))) float smem[C::SMEM];
    const int bid = xcd_remap(blockIdx.x, args.total_tiles);
    GemmProb p;
    int t = bid;
    if (args.nprob > 0) {
        int lo = 0, hi = args.nprob - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (args.tile_begin[mid] <= bid) lo = mid; else hi = mid - 1;
        }
        p = args.probs[lo];
        t = bid - args.tile_begin[lo];
    } else {
        p = args.single;
    }
    int tm, tn;
    raster(t, p.tiles_m, p.tiles_n, tm, tn);
    gemm_tile<C, AT, BT, ABF, BBF, X6>(p, tm, tn, args.alpha_scale, smem);
}

// The X6 products: same problem tables and tiles as gemm_grouped_kernel.
template <class C, bool AT, bool BT, bool ABF, bool BBF>
__global__ __launch_bounds__(C::NT) __attribute__((amdgpu_waves_per_eu(2))) void gemm_x6_kernel(GemmArgs args) {
    __shared__ __attribute__((aligned(16))) char smem[X6Lds<C, ABF, BBF>::BYTES];
    const int bid = xcd_remap(blockIdx.x, args.total_tiles);
    GemmProb p;
    int t = bid;
    if (args.nprob > 0) {
        int lo = 0, hi = args.nprob - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (args.tile_begin[mid] <= bid) lo = mid; else hi = mid - 1;
        }
        p = args.probs[lo];
        t = bid - args.tile_begin[lo];
    } else {
        p = args.single;
    }
    int tm, tn;
    raster(t, p.tiles_m, p.tiles_n, tm, tn);
    gemm_tile_x6<C, AT, BT, ABF, BBF>(p, tm, tn, args.alpha_scale, smem);
}

template <bool AT, bool BT, bool ABF, bool BBF, bool X6 = false>
hipError_t launch(int cfg, const GemmArgs& a, hipStream_t s) {
    if (a.total_tiles <= 0) return hipSuccess;
    if constexpr (X6 && kX6SplitAtFill) {
        if (cfg == 1)
            gemm_x6_kernel<LargeCfg, AT, BT, ABF, BBF><<<dim3(a.total_tiles), dim3(LargeCfg::NT), 0, s>>>(a);
        else
            gemm_x6_kernel<SmallCfg, AT, BT, ABF, BBF><<<dim3(a.total_tiles), dim3(SmallCfg::NT), 0, s>>>(a);
    } else if constexpr (X6 && ABF) {
        return hipErrorInvalidValue;   // the in-register split takes an fp32 A
    } else {
        if (cfg == 1)
            gemm_grouped_kernel<LargeCfg, AT, BT, ABF, BBF, X6><<<dim3(a.total_tiles), dim3(LargeCfg::NT), 0, s>>>(a);
        else
            gemm_grouped_kernel<SmallCfg, AT, BT, ABF, BBF, X6><<<dim3(a.total_tiles), dim3(SmallCfg::NT), 0, s>>>(a);
    }
    return hipGetLastError();
}

}  // namespace

// ---- QR in-block update: C -= Y W2 with Y the unit-lower reflector block ----
//
// At panel p: C = the rest of the outer block, Z[k:, k+jb : block end],
// Y = Z[k:, k:k+jb]; W2 (jb x ncols) comes from qr_reduce.
__global__ __launch_bounds__(QrCfg::NT) void qr_update_kernel(const QrJob* __restrict__ jobs,
                                                            QrClasses C, int p) {
    __shared__ __attribute__((aligned(16))) float smem[QrCfg::SMEM];
    int job, local;
    if (!qr_locate(C, QG_UPDATE, p, blockIdx.x, job, local)) return;
    const QrJob J = jobs[job];
    const int k = p * kQrPB;
    const int jb = min(kQrPB, J.d - k);
    const int L = J.d - k;
    const int ncols = qr_inblock_cols(J.d, p);
    GemmProb g;
    g.A = J.Z + (int64_t)k * J.d + k;
    g.B = J.W2;
    g.C = J.Z + (int64_t)k * J.d + k + jb;
    g.lda = J.d;
    g.ldb = J.d;
    g.ldc = J.d;
    g.M = L;
    g.N = ncols;
    g.K = jb;
    g.flags = (J.d % 4 == 0) ? (GF_A_VEC | GF_B_VEC) : 0u;
    g.alpha = -1.f;
    g.beta = 1.f;
    g.tiles_m = (L + QrCfg::BM - 1) / QrCfg::BM;
    g.tiles_n = (ncols + QrCfg::BN - 1) / QrCfg::BN;
    int tm, tn;
    raster(local, g.tiles_m, g.tiles_n, tm, tn);
    qr_update_tile(g, tm, tn, smem);
}

hipError_t launch_qr_update(const QrJob* jobs, const QrClasses& C, int p, hipStream_t s) {
    const int blocks = qr_total_blocks(C, QG_UPDATE, p);
    if (blocks <= 0) return hipSuccess;
    qr_update_kernel<<<dim3(blocks), dim3(QrCfg::NT), 0, s>>>(jobs, C, p);
    return hipGetLastError();
}

#define MATOPT_VARIANTS(X)                                                                         \
    X(0, false, false, false, false) X(1, true, false, false, false) X(2, false, true, false, false)   \
    X(3, true, true, false, false) X(4, false, false, true, false) X(5, true, false, true, false)      \
    X(6, false, true, true, false) X(7, true, true, true, false) X(8, false, false, false, true)       \
    X(9, true, false, false, true) X(10, false, true, false, true) X(11, true, true, false, true)      \
    X(12, false, false, true, true) X(13, true, false, true, true) X(14, false, true, true, true)      \
    X(15, true, true, true, true)

static hipError_t dispatch(int variant, int cfg, const GemmArgs& a, hipStream_t s) {
    switch (variant) {
#define X(v, at, bt, abf, bbf) \
    case v: return launch<at, bt, abf, bbf>(cfg, a, s);
        MATOPT_VARIANTS(X)
#undef X
        // fp32 products on bf16 MFMAs: the operand variants of the rotations
        // and of the refresh's products
        case GV_X6 | 0: return launch<false, false, false, false, true>(cfg, a, s);
        case GV_X6 | 1: return launch<true, false, false, false, true>(cfg, a, s);
        case GV_X6 | 2: return launch<false, true, false, false, true>(cfg, a, s);
        case GV_X6 | 8: return launch<false, false, false, true, true>(cfg, a, s);
        case GV_X6 | 4: return launch<false, false, true, false, true>(cfg, a, s);
        case GV_X6 | 5: return launch<true, false, true, false, true>(cfg, a, s);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_gemm_grouped(int variant, int cfg, const GemmProb* probs, const int32_t* tile_begin,
                               int nprob, int total_tiles, float alpha_scale, hipStream_t s) {
    if (nprob <= 0) return hipSuccess;
    GemmArgs a{};
    a.probs = probs;
    a.tile_begin = tile_begin;
    a.nprob = nprob;
    a.total_tiles = total_tiles;
    a.alpha_scale = alpha_scale;
    return dispatch(variant, cfg, a, s);
}

hipError_t launch_gemm_single(int variant, int cfg, const GemmProb& prob, hipStream_t s) {
    GemmArgs a{};
    a.nprob = 0;
    a.total_tiles = prob.tiles_m * prob.tiles_n;
    a.alpha_scale = 1.f;
    a.single = prob;
    return dispatch(variant, cfg, a, s);
}

}  // namespace matopt
