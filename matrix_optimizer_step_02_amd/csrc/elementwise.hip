// Multi-tensor elementwise kernels of the step (HBM-bandwidth bound).
//
//  momentum:      M <- beta1 M + (1 - beta1) G          (M fp32 or bf16 RNE)
//  rotated Adam:  v <- beta2 v + (1 - beta2) G~ * G~     (square in fp32)
//                 u  = m~ / (sqrt(v) + eps)              (u overwrites m~)
//
// One launch covers every matrix of a micro-group: the matrices are cut into
// chunks of kEwChunk elements, concatenated in chunk space, and each
// workgroup finds its matrix by a binary search over the chunk offsets. A
// thread moves four 16-byte groups (fp32) per tensor, and for each group the
// 256 threads of the workgroup touch one contiguous 4 KiB span, so every
// access is a full-line, coalesced one.
#include "internal.h"

namespace matopt {

typedef float f32x4 __attribute__((ext_vector_type(4)));

namespace {

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
    return __uint_as_float(((uint32_t)h) << 16);
}

// fp32 -> bf16, round to nearest even; NaN stays a (quiet) NaN, overflow
// rounds to infinity.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x0040u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

__device__ __forceinline__ int find_seg(const EwSeg* segs, int nseg, int64_t chunk) {
    int lo = 0, hi = nseg - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (segs[mid].chunk_begin <= chunk) lo = mid; else hi = mid - 1;
    }
    return lo;
}

__device__ __forceinline__ float ema(float b, float x, float omb, float y) {
    return __builtin_fmaf(b, x, omb * y);
}

__global__ __launch_bounds__(kEwThreads) void momentum_kernel(const EwSeg* __restrict__ segs,
                                                              int nseg, float beta1) {
    const int64_t chunk = blockIdx.x;
    const EwSeg S = segs[find_seg(segs, nseg, chunk)];
    const int64_t base = (chunk - S.chunk_begin) * kEwChunk;
    const float omb = 1.f - beta1;
#pragma unroll
    for (int q = 0; q < kEwPerThread / 4; ++q) {
        const int64_t i = base + 4 * ((int64_t)q * kEwThreads + threadIdx.x);
        if (i >= S.n) break;
        if (S.vec && i + 3 < S.n) {
            const f32x4 g = *(const f32x4*)(S.a + i);
            if (S.b_bf16) {
                uint2 raw = *(const uint2*)((const uint16_t*)S.b + i);
                f32x4 m;
                m[0] = __uint_as_float(raw.x << 16);
                m[1] = __uint_as_float(raw.x & 0xffff0000u);
                m[2] = __uint_as_float(raw.y << 16);
                m[3] = __uint_as_float(raw.y & 0xffff0000u);
                uint16_t o[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) o[e] = f32_to_bf16(ema(beta1, m[e], omb, g[e]));
                uint2 w;
                w.x = (uint32_t)o[0] | ((uint32_t)o[1] << 16);
                w.y = (uint32_t)o[2] | ((uint32_t)o[3] << 16);
                *(uint2*)((uint16_t*)S.b + i) = w;
            } else {
                f32x4 m = *(const f32x4*)((const float*)S.b + i);
#pragma unroll
                for (int e = 0; e < 4; ++e) m[e] = ema(beta1, m[e], omb, g[e]);
                *(f32x4*)((float*)S.b + i) = m;
            }
        } else {
            for (int e = 0; e < 4 && i + e < S.n; ++e) {
                const float g = S.a[i + e];
                if (S.b_bf16) {
                    uint16_t* p = (uint16_t*)S.b + i + e;
                    *p = f32_to_bf16(ema(beta1, bf16_to_f32(*p), omb, g));
                } else {
                    float* p = (float*)S.b + i + e;
                    *p = ema(beta1, *p, omb, g);
                }
            }
        }
    }
}

__device__ __forceinline__ void adam1(float g, float m, float& v, float& u, float beta2, float omb2,
                                      float eps) {
    const float g2 = g * g;
    v = __builtin_fmaf(beta2, v, omb2 * g2);
    u = m / (__builtin_sqrtf(v) + eps);
}

__global__ __launch_bounds__(kEwThreads) void rotated_adam_kernel(const EwSeg* __restrict__ segs,
                                                                  int nseg, float beta2, float eps) {
    const int64_t chunk = blockIdx.x;
    const EwSeg S = segs[find_seg(segs, nseg, chunk)];
    const int64_t base = (chunk - S.chunk_begin) * kEwChunk;
    const float omb2 = 1.f - beta2;
    float* mu = (float*)S.b;
#pragma unroll
    for (int q = 0; q < kEwPerThread / 4; ++q) {
        const int64_t i = base + 4 * ((int64_t)q * kEwThreads + threadIdx.x);
        if (i >= S.n) break;
        if (S.vec && i + 3 < S.n) {
            const f32x4 g = *(const f32x4*)(S.a + i);
            const f32x4 m = *(const f32x4*)(mu + i);
            const f32x4 v0 = *(const f32x4*)(S.c + i);
            f32x4 v, u;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float ve = v0[e], ue;
                adam1(g[e], m[e], ve, ue, beta2, omb2, eps);
                v[e] = ve;
                u[e] = ue;
            }
            *(f32x4*)(S.c + i) = v;
            *(f32x4*)(mu + i) = u;
        } else {
            for (int e = 0; e < 4 && i + e < S.n; ++e) {
                float v = S.c[i + e], u;
                adam1(S.a[i + e], mu[i + e], v, u, beta2, omb2, eps);
                S.c[i + e] = v;
                mu[i + e] = u;
            }
        }
    }
}

}  // namespace

hipError_t launch_momentum(const EwSeg* segs, int nseg, int64_t total_chunks, float beta1,
                           hipStream_t s) {
    if (nseg <= 0 || total_chunks <= 0) return hipSuccess;
    hipLaunchKernelGGL(momentum_kernel, dim3((unsigned)total_chunks), dim3(kEwThreads), 0, s, segs,
                       nseg, beta1);
    return hipGetLastError();
}

hipError_t launch_rotated_adam(const EwSeg* segs, int nseg, int64_t total_chunks, float beta2,
                               float eps, hipStream_t s) {
    if (nseg <= 0 || total_chunks <= 0) return hipSuccess;
    hipLaunchKernelGGL(rotated_adam_kernel, dim3((unsigned)total_chunks), dim3(kEwThreads), 0, s,
                       segs, nseg, beta2, eps);
    return hipGetLastError();
}

}  // namespace matopt
