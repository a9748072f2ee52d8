// Device structures of the orthogonalised-momentum step (OPT_FLAG_MUON): the
// momentum's orthogonal polar factor by Newton-Schulz iteration, then
// W <- W - lr O.
#pragma once

#include "internal.h"

namespace matopt {

// One matrix of the orthogonalisation's elementwise launches, cut into
// chunks of kEwChunk elements like EwSeg. X and P are m x n fp32 scratch (the
// iterate and X times its Gram matrix), `slot` the matrix's entry in the
// group's norm array.
struct MuonSeg {
    const void* M;
    float* X;
    const float* P;
    float* W;
    int64_t n;
    int64_t chunk_begin;
    int32_t m_bf16;
    int32_t slot;
};

// part[c] = sum of M^2 over chunk c (float64); inv[slot] = 1 / ||M||_F from a
// matrix's partials in order (0 for a zero matrix); X = inv M.
hipError_t launch_muon_norm(const MuonSeg* segs, int nseg, int64_t chunks, double* part, float* inv,
                            hipStream_t s);
hipError_t launch_muon_scale(const MuonSeg* segs, int nseg, int64_t chunks, const float* inv, hipStream_t s);
// X <- 1.5 X - 0.5 P, or for the last iteration W <- W - lr (1.5 X - 0.5 P).
hipError_t launch_muon_combine(const MuonSeg* segs, int nseg, int64_t chunks, bool last, float lr,
                               hipStream_t s);

}  // namespace matopt
