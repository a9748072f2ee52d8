// Elementwise kernels of the orthogonalised-momentum step (HBM-bound): the
// Frobenius norm of each momentum matrix, the starting iterate
// X_0 = M / ||M||_F, and the Newton-Schulz combination X <- 1.5 X - 0.5 P,
// whose last application is fused with the weight update W <- W - lr X.
// The Gram products P = X (X^T X) (or (X X^T) X) run on the grouped GEMM.
//
// Launches cover a micro-group in chunk space (as the other elementwise
// kernels); each thread walks its chunk with a stride of the workgroup size,
// so every access is coalesced. The norm is deterministic: per-chunk float64
// partials, then one workgroup per matrix sums them in a fixed order.
#include "variant_muon.h"

namespace matopt {

namespace {

constexpr int NT = kEwThreads;

__device__ __forceinline__ int find_muon_seg(const MuonSeg* segs, int nseg, int64_t chunk) {
    int lo = 0, hi = nseg - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (segs[mid].chunk_begin <= chunk) lo = mid; else hi = mid - 1;
    }
    return lo;
}

__device__ __forceinline__ float load_m(const MuonSeg& S, int64_t e) {
    if (S.m_bf16) return __uint_as_float(((uint32_t)gptr((const uint16_t*)S.M)[e]) << 16);
    return gptr((const float*)S.M)[e];
}

// Sum over the workgroup, in a fixed order; the result is valid in thread 0.
__device__ __forceinline__ double block_sum(double x) {
    __shared__ double red[NT / 64];
    for (int o = 32; o > 0; o >>= 1) x += __shfl_down(x, o);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
    __syncthreads();
    double t = 0.0;
    if (threadIdx.x == 0)
        for (int w = 0; w < NT / 64; ++w) t += red[w];
    return t;
}

__global__ __launch_bounds__(NT) void muon_sumsq_kernel(const MuonSeg* __restrict__ segs, int nseg,
                                                        double* __restrict__ part) {
    const int64_t chunk = blockIdx.x;
    const MuonSeg S = segs[find_muon_seg(segs, nseg, chunk)];
    const int64_t base = (chunk - S.chunk_begin) * kEwChunk;
    double acc = 0.0;
    for (int q = 0; q < kEwPerThread; ++q) {
        const int64_t e = base + (int64_t)q * NT + threadIdx.x;
        if (e >= S.n) break;
        const double x = load_m(S, e);
        acc += x * x;
    }
    const double t = block_sum(acc);
    if (threadIdx.x == 0) gptr(part)[chunk] = t;
}

__global__ __launch_bounds__(NT) void muon_inv_norm_kernel(const MuonSeg* __restrict__ segs,
                                                           const double* __restrict__ part,
                                                           float* __restrict__ inv) {
    const MuonSeg S = segs[blockIdx.x];
    const int64_t nch = (S.n + kEwChunk - 1) / kEwChunk;
    double acc = 0.0;
    for (int64_t c = threadIdx.x; c < nch; c += NT) acc += gptr(part)[S.chunk_begin + c];
    const double t = block_sum(acc);
    if (threadIdx.x == 0) gptr(inv)[S.slot] = t > 0.0 ? (float)(1.0 / sqrt(t)) : 0.f;
}

__global__ __launch_bounds__(NT) void muon_scale_kernel(const MuonSeg* __restrict__ segs, int nseg,
                                                        const float* __restrict__ inv) {
    const int64_t chunk = blockIdx.x;
    const MuonSeg S = segs[find_muon_seg(segs, nseg, chunk)];
    const int64_t base = (chunk - S.chunk_begin) * kEwChunk;
    const float f = gptr(inv)[S.slot];
    for (int q = 0; q < kEwPerThread; ++q) {
        const int64_t e = base + (int64_t)q * NT + threadIdx.x;
        if (e >= S.n) break;
        gptr(S.X)[e] = load_m(S, e) * f;
    }
}

__global__ __launch_bounds__(NT) void muon_combine_kernel(const MuonSeg* __restrict__ segs, int nseg, int last,
                                                          float lr) {
    const int64_t chunk = blockIdx.x;
    const MuonSeg S = segs[find_muon_seg(segs, nseg, chunk)];
    const int64_t base = (chunk - S.chunk_begin) * kEwChunk;
    for (int q = 0; q < kEwPerThread; ++q) {
        const int64_t e = base + (int64_t)q * NT + threadIdx.x;
        if (e >= S.n) break;
        const float x = __builtin_fmaf(1.5f, gptr(S.X)[e], -0.5f * gptr(S.P)[e]);
        if (last) gptr(S.W)[e] = __builtin_fmaf(-lr, x, gptr(S.W)[e]);
        else      gptr(S.X)[e] = x;
    }
}

}  // namespace

hipError_t launch_muon_norm(const MuonSeg* segs, int nseg, int64_t chunks, double* part, float* inv,
                            hipStream_t s) {
    if (nseg <= 0 || chunks <= 0) return hipSuccess;
    hipLaunchKernelGGL(muon_sumsq_kernel, dim3((unsigned)chunks), dim3(NT), 0, s, segs, nseg, part);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(muon_inv_norm_kernel, dim3(nseg), dim3(NT), 0, s, segs, part, inv);
    return hipGetLastError();
}

hipError_t launch_muon_scale(const MuonSeg* segs, int nseg, int64_t chunks, const float* inv, hipStream_t s) {
    if (nseg <= 0 || chunks <= 0) return hipSuccess;
    hipLaunchKernelGGL(muon_scale_kernel, dim3((unsigned)chunks), dim3(NT), 0, s, segs, nseg, inv);
    return hipGetLastError();
}

hipError_t launch_muon_combine(const MuonSeg* segs, int nseg, int64_t chunks, bool last, float lr,
                               hipStream_t s) {
    if (nseg <= 0 || chunks <= 0) return hipSuccess;
    hipLaunchKernelGGL(muon_combine_kernel, dim3((unsigned)chunks), dim3(NT), 0, s, segs, nseg, last ? 1 : 0, lr);
    return hipGetLastError();
}

}  // namespace matopt
