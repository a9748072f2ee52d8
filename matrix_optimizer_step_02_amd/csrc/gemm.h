// Declarations of the grouped fp32 GEMM (csrc/gemm.hip): the problem
// descriptor, the operand variants, the tile configurations and the launches.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gmem.h"

namespace matopt {

// ---------------------------------------------------------------- GEMM ----

enum : uint32_t {
    GF_A_VEC = 1u << 0,   // A: ld % 4 == 0 and 16-byte (fp32) / 8-byte (bf16) aligned base
    GF_B_VEC = 1u << 1,
};

// One product C = alpha * alpha_scale * op(A) op(B) + beta * C. The launch's
// template fixes whether A is stored K x M (transposed) and B stored N x K.
struct GemmProb {
    const void* A;
    const void* B;
    float* C;
    int64_t lda, ldb, ldc;
    int32_t M, N, K;
    uint32_t flags;
    float alpha, beta;
    int32_t tiles_m, tiles_n;
};

// Launch variant: bit 0 A stored K x M (transposed), bit 1 B stored N x K,
// bit 2 A is bfloat16, bit 3 B is bfloat16. All problems of one grouped
// launch share the variant.
inline int gemm_variant(bool at, bool bt, bool a_bf16, bool b_bf16) {
    return (at ? 1 : 0) | (bt ? 2 : 0) | (a_bf16 ? 4 : 0) | (b_bf16 ? 8 : 0);
}
// Bit 4: the fp32 product runs on bf16 MFMAs, each operand split into three
// exact bf16 pieces and six piece products kept (fp32 accuracy; three when
// one operand is bf16, which is its own high piece). Available for the
// variants 0 (A M x K, B K x N), 1 (A stored K x M), 2 (B stored N x K),
// 8 (B bf16), and 4 and 5 (A bf16, as stored or transposed; not with the
// in-register split that MATOPT_X6_REGISTER_SPLIT selects).
#ifdef MATOPT_X6_REGISTER_SPLIT
constexpr bool kX6SplitAtFill = false;
#else
constexpr bool kX6SplitAtFill = true;
#endif
constexpr int GV_X6 = 16;
inline bool gemm_x6_available(int variant) {
    return variant == 0 || variant == 1 || variant == 2 || variant == 8 ||
           (kX6SplitAtFill && (variant == 4 || variant == 5));
}

// Two tile configurations of the grouped GEMM (rotations, Gram products,
// opt_gemm): 128x128 outputs per workgroup of 2x2 wavefronts (64x64 each),
// and 256x256 per workgroup of 2x4 wavefronts (128x64 each), which reuses
// every staged operand more but needs many tiles to fill the GPU. A launch
// takes the large tiles when it has at least kGemmLargeMinTiles of them.
struct GemmTileCfg {
    int bm, bn;
};
#ifndef MATOPT_LARGE_BM
#define MATOPT_LARGE_BM 256
#define MATOPT_LARGE_BN 256
#endif
constexpr GemmTileCfg kGemmCfgs[2] = {{128, 128}, {MATOPT_LARGE_BM, MATOPT_LARGE_BN}};
constexpr int kGemmLargeMinTiles = 512;
constexpr int kQrTile = 128;   // output tile of the QR trailing update

// Grouped launch over `nprob` problems laid out back to back in tile space;
// tile_begin[p] is the first tile of problem p (ascending, tile_begin[0] = 0).
// `cfg` indexes kGemmCfgs; every problem's tiles_m/tiles_n must use it.
hipError_t launch_gemm_grouped(int variant, int cfg, const GemmProb* probs, const int32_t* tile_begin,
                               int nprob, int total_tiles, float alpha_scale, hipStream_t s);
hipError_t launch_gemm_single(int variant, int cfg, const GemmProb& prob, hipStream_t s);

}  // namespace matopt
