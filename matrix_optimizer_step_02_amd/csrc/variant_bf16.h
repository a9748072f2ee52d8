// Device structures of the bf16-rotation variant: the rotations run on
// bfloat16 operands (v_mfma_f32_32x32x16_bf16, binary32 accumulation), with
// bfloat16 copies of the bases kept in the workspace between refreshes.
#pragma once

#include "internal.h"

namespace matopt {

// ------------------------------------------------------- bf16 GEMM (NT) ----

// C = alpha * alpha_scale * A B^T + beta C with A (M x K) and B (N x K) bf16,
// both row-major with k contiguous. Requirements checked by the host: K, lda
// and ldb multiples of 8, A and B 16-byte aligned (every 8-element group of
// k is one 16-byte load). C is fp32 (ldc) or, for c_bf16 launches, bf16
// rounded to nearest even with beta = 0; a bf16 C also gets zeros in columns
// [N, pad_n) of each row (the zero k padding of a later product's operand).
//
// Pieced products. The k range can be a sum of `np` periods: the product is
// sum_{q < np} A_q B_q^T with A_q = A + q a_ps and B_q = B + q b_ps (element
// offsets), each over the same K. An operand with a piece stride of 0 is
// read again in every period. This is how an fp32 operand split into three
// exact bf16 pieces (hi, mid, lo) meets a bf16 operand in one accumulation
// chain. Each period starts on a 64-aligned slab (kper = K rounded up to 64);
// np = 1 with zero piece strides is the plain product.
struct Gemm16Prob {
    const uint16_t* A;
    const uint16_t* B;
    void* C;
    int64_t lda, ldb, ldc;
    int64_t a_ps, b_ps;
    int32_t M, N, K;
    int32_t np, kper;
    int32_t pad_n;
    float alpha, beta;
    int32_t tiles_m, tiles_n;
};

// Tile configurations: 128 x 128 (2 x 2 wavefronts of 64 x 64) and 256 x 256
// (2 x 2 wavefronts of 128 x 128). A launch takes the large tiles when it has
// at least kGemm16LargeMinTiles of them.
constexpr GemmTileCfg kGemm16Cfgs[2] = {{128, 128}, {256, 256}};
constexpr int kGemm16LargeMinTiles = 256;

hipError_t launch_gemm16_grouped(bool c_bf16, int cfg, const Gemm16Prob* probs, const int32_t* tile_begin,
                                 int nprob, int total_tiles, float alpha_scale, hipStream_t s);
hipError_t launch_gemm16_single(bool c_bf16, int cfg, const Gemm16Prob& prob, hipStream_t s);

// ---------------------------------------------------------- elementwise ----

// One matrix of the variant's elementwise launches (chunked like EwSeg).
//  momentum: a = G, b = M (fp32 or bf16, updated); o1 = bf16 copy of G,
//            o2 = bf16 copy of the new M (NULL when M is bf16 and the
//            rotation reads it directly).
//  Adam:     a = G~, b = m~, c = v (updated); o1 = u rounded to bf16; with
//            carry, first b <- beta1 b + (1 - beta1) a (the carried m~, fp32).
// The bf16 outputs are row-major with the row stride equal to the number of
// columns, so the vector path needs n % 8 == 0; other shapes take EwSeg
// launches and a pack to a padded layout.
struct Ew16Seg {
    const float* a;
    void* b;
    float* c;
    uint16_t* o1;
    uint16_t* o2;
    int64_t n;
    int64_t chunk_begin;
    int32_t b_bf16;
    int32_t vec;
    int32_t carry;
};

hipError_t launch_momentum16(const Ew16Seg* segs, int nseg, int64_t total_chunks, float beta1, hipStream_t s);
// The bf16 copies of G and M (as stored) alone, for a step whose refresh ran
// between the momentum update and the rotations.
hipError_t launch_convert16(const Ew16Seg* segs, int nseg, int64_t total_chunks, hipStream_t s);
hipError_t launch_adam16(const Ew16Seg* segs, int nseg, int64_t total_chunks, float beta1, float beta2, float eps,
                         hipStream_t s);

// Rows x cols of an fp32 or bf16 matrix (row stride ld_src) to bf16 with row
// stride ld_dst >= cols, zeros in columns [cols, ld_dst).
struct PackJob {
    const void* src;
    uint16_t* dst;
    int64_t rows, cols, ld_src, ld_dst;
    int64_t chunk_begin;
    int32_t src_bf16;
};
hipError_t launch_pack16(const PackJob* jobs, int njobs, int64_t total_chunks, hipStream_t s);

// A d x d fp32 basis X to bf16 copies Xb = X and Xt = X^T, both d x dp
// (dp = d rounded up to 8) with zero columns [d, dp). 32 x 32 tiles over
// dp x dp; tile_begin is the job's first tile.
struct BasisJob {
    const void* X;      // fp32, or bf16 with x_bf16 (bases stored in 16 bits)
    uint16_t* Xb;       // NULL: no row-padded copy (X itself serves, bf16 with d == dp)
    uint16_t* Xt;
    int32_t d, dp;
    int32_t tile_begin;
    int32_t x_bf16;
};
constexpr int kBasisTile = 32;
hipError_t launch_basis16(const BasisJob* jobs, int njobs, int total_tiles, hipStream_t s);

// Bases stored in 16 bits: n elements between a bf16 basis and its fp32
// working copy in the refresh scratch. to16 = 0 widens (exact), 1 rounds to
// nearest even. Jobs are laid out back to back in chunks of kEwChunk.
struct CvtJob {
    const void* src;
    void* dst;
    int64_t n;
    int64_t chunk_begin;
    int32_t to16;
};
hipError_t launch_cvt16(const CvtJob* jobs, int njobs, int64_t total_chunks, hipStream_t s);

// Transposed bf16 pieces of a rows x cols block X (fp32 or bf16, row stride
// ld_src): dst + p * piece_stride holds piece p as a cols x ld_dst row-major
// matrix, dst_p[c][k] = piece_p(X[k][c]) for k < rows, zeros for rows <= k <
// ld_dst. With npieces == 3 (fp32 X) the pieces are hi = rb(x),
// mid = rb(x - hi), lo = x - hi - mid, which sum to x exactly (each residual
// is exact in fp32 and lo fits in bf16), so a product with X equals the sum of
// three bf16 products up to fp32 accumulation; with npieces == 1 the single
// piece is rb(x) (an exact transpose for bf16 X). 32 x 32 tiles over
// ld_dst x cols; tile_begin is the job's first tile.
struct SplitJob {
    const void* src;
    uint16_t* dst;
    int64_t ld_src, ld_dst, piece_stride;
    int32_t rows, cols;
    int32_t npieces, src_bf16;
    int32_t tile_begin;
};
hipError_t launch_split16(const SplitJob* jobs, int njobs, int total_tiles, hipStream_t s);

}  // namespace matopt
