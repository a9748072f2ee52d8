// State checks and basis re-orthonormalisation.
//
// Checks the pages prescribe for a rotated-basis optimizer: the rotation
// matrices must stay orthogonal (U^T U = I; the Pipeline-parallelism page,
// section 5.1), and the second moment is suspect when std(v) / mean(|v|)
// exceeds 10 or when its minimum is not positive where it divides (the
// three-layer decoupling page, sections 4.3 and 4.4). The statistics of v
// and the count of non-finite entries of W, M and v come from one scan per
// micro-group, reduced per chunk and then per matrix in a fixed order, in
// float64. The drifts max |X^T X - I| read the Gram matrices X^T X, formed
// by the grouped GEMM. Re-orthonormalisation (section 5.1 again: X (X^T
// X)^(-1/2), the polar factor) runs Newton-Schulz steps X <- 1.5 X - 0.5 X
// (X^T X), whose products are grouped GEMMs; the combine step is here.
#include "internal.h"

namespace matopt {

typedef float f32x4 __attribute__((ext_vector_type(4)));

namespace {

constexpr int NT = kEwThreads;
constexpr int NQ = kEwPerThread / 4;

__device__ __forceinline__ bool finite(float x) { return __builtin_isfinite(x); }

__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float(((uint32_t)h) << 16); }

// Workgroup reduction of a partial record (fixed tree: wavefront butterfly,
// then the four wavefronts in order). Every thread gets the result.
__device__ HealthPartial block_reduce(HealthPartial x) {
    __shared__ HealthPartial sh[NT / 64];
    for (int m = 32; m >= 1; m >>= 1) {
        x.sabs += __shfl_xor(x.sabs, m, 64);
        x.s += __shfl_xor(x.s, m, 64);
        x.s2 += __shfl_xor(x.s2, m, 64);
        x.vmin = fminf(x.vmin, __shfl_xor(x.vmin, m, 64));
        x.vmax = fmaxf(x.vmax, __shfl_xor(x.vmax, m, 64));
        x.nonfinite += __shfl_xor(x.nonfinite, m, 64);
    }
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) sh[wave] = x;
    __syncthreads();
    HealthPartial r = sh[0];
    for (int w = 1; w < NT / 64; ++w) {
        r.sabs += sh[w].sabs;
        r.s += sh[w].s;
        r.s2 += sh[w].s2;
        r.vmin = fminf(r.vmin, sh[w].vmin);
        r.vmax = fmaxf(r.vmax, sh[w].vmax);
        r.nonfinite += sh[w].nonfinite;
    }
    __syncthreads();
    return r;
}

__device__ __forceinline__ int find_seg(const HealthSeg* segs, int nseg, int64_t chunk) {
    int lo = 0, hi = nseg - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (segs[mid].chunk_begin <= chunk) lo = mid; else hi = mid - 1;
    }
    return lo;
}

__global__ __launch_bounds__(NT) void health_clear_kernel(HealthOut* out, int n) {
    const int i = blockIdx.x * NT + threadIdx.x;
    if (i >= n) return;
    HealthOut z{};
    z.vmin = __builtin_inff();
    z.vmax = -__builtin_inff();
    out[i] = z;
}

// One chunk of kEwChunk elements of one matrix per workgroup. NaN in v makes
// the sums NaN; fminf/fmaxf skip it (it is counted as non-finite).
__global__ __launch_bounds__(NT) void health_partials_kernel(const HealthSeg* __restrict__ segs, int nseg,
                                                             HealthPartial* __restrict__ part) {
    const int64_t chunk = blockIdx.x;
    const HealthSeg S = segs[find_seg(segs, nseg, chunk)];
    const int64_t base = (chunk - S.chunk_begin) * kEwChunk;
    HealthPartial x{0.0, 0.0, 0.0, __builtin_inff(), -__builtin_inff(), 0};
    gmem<const float> W = gptr(S.W);
    gmem<const float> V = gptr(S.v);
    for (int q = 0; q < kEwPerThread; ++q) {
        const int64_t i = base + (int64_t)q * NT + threadIdx.x;
        if (i >= S.n) break;
        const float v = V[i], w = W[i];
        const float m = S.m_bf16 ? bf16_to_f32(gptr((const uint16_t*)S.M)[i]) : gptr((const float*)S.M)[i];
        x.sabs += fabs((double)v);
        x.s += (double)v;
        x.s2 += (double)v * (double)v;
        x.vmin = fminf(x.vmin, v);
        x.vmax = fmaxf(x.vmax, v);
        x.nonfinite += !finite(v) + !finite(w) + !finite(m);
    }
    const HealthPartial r = block_reduce(x);
    if (threadIdx.x == 0) part[chunk] = r;
}

// One workgroup per matrix: its chunks' partials, strided over the threads,
// then the workgroup tree.
__global__ __launch_bounds__(NT) void health_final_kernel(const HealthSeg* __restrict__ segs,
                                                          const HealthPartial* __restrict__ part,
                                                          HealthOut* __restrict__ out) {
    const HealthSeg S = segs[blockIdx.x];
    const int64_t nch = (S.n + kEwChunk - 1) / kEwChunk;
    HealthPartial x{0.0, 0.0, 0.0, __builtin_inff(), -__builtin_inff(), 0};
    for (int64_t c = threadIdx.x; c < nch; c += NT) {
        const HealthPartial p = part[S.chunk_begin + c];
        x.sabs += p.sabs;
        x.s += p.s;
        x.s2 += p.s2;
        x.vmin = fminf(x.vmin, p.vmin);
        x.vmax = fmaxf(x.vmax, p.vmax);
        x.nonfinite += p.nonfinite;
    }
    const HealthPartial r = block_reduce(x);
    if (threadIdx.x == 0) {
        HealthOut& o = out[S.out];
        o.sabs = r.sabs;
        o.s = r.s;
        o.s2 = r.s2;
        o.vmin = r.vmin;
        o.vmax = r.vmax;
        o.nonfinite = r.nonfinite;
        o.n = S.n;
    }
}

// max |G - I| over one chunk of G per workgroup; NaN counts as the largest.
__global__ __launch_bounds__(NT) void drift_kernel(const DriftJob* __restrict__ jobs, HealthOut* out) {
    const DriftJob J = jobs[blockIdx.y];
    const int64_t d = J.d, n = d * d;
    const int64_t base = (int64_t)blockIdx.x * kEwChunk;
    if (base >= n) return;
    gmem<const float> G = gptr(J.G);
    uint32_t worst = 0;
    for (int q = 0; q < kEwPerThread; ++q) {
        const int64_t e = base + (int64_t)q * NT + threadIdx.x;
        if (e >= n) break;
        const int64_t i = e / d, j = e - i * d;
        const float dev = fabsf(G[e] - (i == j ? 1.f : 0.f));
        const uint32_t bits = finite(dev) ? __float_as_uint(dev) : 0x7f800000u;
        worst = bits > worst ? bits : worst;
    }
    for (int m = 32; m >= 1; m >>= 1) {
        const uint32_t o = __shfl_xor(worst, m, 64);
        worst = o > worst ? o : worst;
    }
    if ((threadIdx.x & 63) == 0)
        atomicMax(J.which ? &out[J.out].drift_v : &out[J.out].drift_u, worst);
}

__global__ __launch_bounds__(NT) void ns_combine_kernel(const NsJob* __restrict__ jobs) {
    const NsJob J = jobs[blockIdx.y];
    const int64_t base = (int64_t)blockIdx.x * kEwChunk;
    gmem<float> X = gptr(J.X);
    gmem<const float> P = gptr(J.P);
    for (int q = 0; q < kEwPerThread; ++q) {
        const int64_t e = base + (int64_t)q * NT + threadIdx.x;
        if (e >= J.n) break;
        X[e] = __builtin_fmaf(1.5f, X[e], -0.5f * P[e]);
    }
}

}  // namespace

hipError_t launch_health_clear(HealthOut* out, int n, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(health_clear_kernel, dim3((n + NT - 1) / NT), dim3(NT), 0, s, out, n);
    return hipGetLastError();
}

hipError_t launch_health_partials(const HealthSeg* segs, int nseg, int64_t chunks, HealthPartial* part,
                                  hipStream_t s) {
    if (nseg <= 0 || chunks <= 0) return hipSuccess;
    hipLaunchKernelGGL(health_partials_kernel, dim3((unsigned)chunks), dim3(NT), 0, s, segs, nseg, part);
    return hipGetLastError();
}

hipError_t launch_health_final(const HealthSeg* segs, int nseg, const HealthPartial* part, HealthOut* out,
                               hipStream_t s) {
    if (nseg <= 0) return hipSuccess;
    hipLaunchKernelGGL(health_final_kernel, dim3(nseg), dim3(NT), 0, s, segs, part, out);
    return hipGetLastError();
}

hipError_t launch_drift(const DriftJob* jobs, int njobs, int max_d, HealthOut* out, hipStream_t s) {
    if (njobs <= 0) return hipSuccess;
    const int64_t n = (int64_t)max_d * max_d;
    hipLaunchKernelGGL(drift_kernel, dim3((unsigned)((n + kEwChunk - 1) / kEwChunk), njobs), dim3(NT), 0, s,
                       jobs, out);
    return hipGetLastError();
}

hipError_t launch_ns_combine(const NsJob* jobs, int njobs, int64_t max_n, hipStream_t s) {
    if (njobs <= 0 || max_n <= 0) return hipSuccess;
    hipLaunchKernelGGL(ns_combine_kernel, dim3((unsigned)((max_n + kEwChunk - 1) / kEwChunk), njobs), dim3(NT), 0,
                       s, jobs);
    return hipGetLastError();
}

}  // namespace matopt
