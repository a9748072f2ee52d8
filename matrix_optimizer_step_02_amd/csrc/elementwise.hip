// Multi-tensor elementwise kernels of the step (HBM-bandwidth bound).
//
//  momentum:      M <- beta1 M + (1 - beta1) G          (M fp32 or bf16 RNE)
//  rotated Adam:  v <- beta2 v + (1 - beta2) G~ * G~     (square in fp32)
//                 u  = m~ / (sqrt(v) + eps)              (u overwrites m~, or to its own buffer)
//                 with the carried rotated momentum first m~ <- beta1 m~ + (1 - beta1) G~
//
// and for the bf16-rotation variant the same two updates with bf16 side
// outputs (G and M rounded for the rotations, u rounded), the conversion of
// the bases to bf16 copies (row-major and transposed) and a pack of a
// matrix to bf16 with a padded row stride.
//
// One launch covers every matrix of a micro-group: the matrices are cut into
// chunks of kEwChunk elements, concatenated in chunk space, and each
// workgroup finds its matrix by a binary search over the chunk offsets. A
// thread moves four 16-byte groups (fp32) per tensor, and for each group the
// 256 threads of the workgroup touch one contiguous 4 KiB span, so every
// access is a full-line, coalesced one.
#include "variant_bf16.h"

namespace matopt {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

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

constexpr int NQ = kEwPerThread / 4;   // 16-byte groups per thread and tensor

__device__ __forceinline__ f32x4 widen_bf16x4(u32x2 raw) {
    f32x4 m;
    m[0] = __uint_as_float(raw.x << 16);
    m[1] = __uint_as_float(raw.x & 0xffff0000u);
    m[2] = __uint_as_float(raw.y << 16);
    m[3] = __uint_as_float(raw.y & 0xffff0000u);
    return m;
}

// Full, aligned chunks take the vector path, which issues every load of the
// thread before the first store (the compiler cannot reorder them itself, as
// the tensors might alias); a ragged or unaligned chunk goes element by
// element.
__global__ __launch_bounds__(kEwThreads) void momentum_kernel(const EwSeg* __restrict__ segs,
                                                              int nseg, float beta1) {
    const int64_t chunk = blockIdx.x;
    const EwSeg S = segs[find_seg(segs, nseg, chunk)];
    const int64_t base = (chunk - S.chunk_begin) * kEwChunk;
    const float omb = 1.f - beta1;
    gmem<const float> G = gptr(S.a);
    if (S.vec && base + kEwChunk <= S.n) {
        f32x4 g[NQ];
#pragma unroll
        for (int q = 0; q < NQ; ++q)
            g[q] = *gptr((const f32x4*)(S.a + base + 4 * (q * kEwThreads + threadIdx.x)));
        if (S.b_bf16) {
            uint16_t* M = (uint16_t*)S.b + base;
            u32x2 raw[NQ];
#pragma unroll
            for (int q = 0; q < NQ; ++q) raw[q] = *gptr((const u32x2*)(M + 4 * (q * kEwThreads + threadIdx.x)));
#pragma unroll
            for (int q = 0; q < NQ; ++q) {
                const f32x4 m = widen_bf16x4(raw[q]);
                uint32_t o[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) o[e] = f32_to_bf16(ema(beta1, m[e], omb, g[q][e]));
                u32x2 w;
                w.x = o[0] | (o[1] << 16);
                w.y = o[2] | (o[3] << 16);
                *gptr((u32x2*)(M + 4 * (q * kEwThreads + threadIdx.x))) = w;
            }
        } else {
            float* M = (float*)S.b + base;
            f32x4 m[NQ];
#pragma unroll
            for (int q = 0; q < NQ; ++q) m[q] = *gptr((const f32x4*)(M + 4 * (q * kEwThreads + threadIdx.x)));
#pragma unroll
            for (int q = 0; q < NQ; ++q) {
#pragma unroll
                for (int e = 0; e < 4; ++e) m[q][e] = ema(beta1, m[q][e], omb, g[q][e]);
                *gptr((f32x4*)(M + 4 * (q * kEwThreads + threadIdx.x))) = m[q];
            }
        }
        return;
    }
    for (int q = 0; q < NQ; ++q) {
        const int64_t i = base + 4 * ((int64_t)q * kEwThreads + threadIdx.x);
        for (int e = 0; e < 4 && i + e < S.n; ++e) {
            const float g = G[i + e];
            if (S.b_bf16) {
                gmem<uint16_t> p = gptr((uint16_t*)S.b + i + e);
                *p = f32_to_bf16(ema(beta1, bf16_to_f32(*p), omb, g));
            } else {
                gmem<float> p = gptr((float*)S.b + i + e);
                *p = ema(beta1, *p, omb, g);
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

// u goes to d when it is set, else over m~ in b. With carry, m~ is first
// advanced in place: b <- beta1 b + (1 - beta1) G~ (the rotated momentum
// carried across a basis epoch), and u uses the new value.
__global__ __launch_bounds__(kEwThreads) void rotated_adam_kernel(const EwSeg* __restrict__ segs,
                                                                  int nseg, float beta1, float beta2,
                                                                  float eps) {
    const int64_t chunk = blockIdx.x;
    const EwSeg S = segs[find_seg(segs, nseg, chunk)];
    const int64_t base = (chunk - S.chunk_begin) * kEwChunk;
    const float omb1 = 1.f - beta1, omb2 = 1.f - beta2;
    if (S.vec && base + kEwChunk <= S.n) {
        const float* Gt = S.a + base;
        float* mb = (float*)S.b + base;
        float* V = S.c + base;
        float* uo = S.d ? S.d + base : mb;
        f32x4 g[NQ], m[NQ], v[NQ];
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            const int o = 4 * (q * kEwThreads + threadIdx.x);
            g[q] = *gptr((const f32x4*)(Gt + o));
            m[q] = *gptr((const f32x4*)(mb + o));
            v[q] = *gptr((const f32x4*)(V + o));
        }
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            const int o = 4 * (q * kEwThreads + threadIdx.x);
            f32x4 u;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                if (S.carry) m[q][e] = ema(beta1, m[q][e], omb1, g[q][e]);
                float ve = v[q][e], ue;
                adam1(g[q][e], m[q][e], ve, ue, beta2, omb2, eps);
                v[q][e] = ve;
                u[e] = ue;
            }
            *gptr((f32x4*)(V + o)) = v[q];
            if (S.carry) *gptr((f32x4*)(mb + o)) = m[q];
            *gptr((f32x4*)(uo + o)) = u;
        }
        return;
    }
    gmem<const float> Gt = gptr(S.a);
    gmem<float> mb = gptr((float*)S.b);
    gmem<float> V = gptr(S.c);
    gmem<float> uo = gptr(S.d ? S.d : (float*)S.b);
    for (int q = 0; q < NQ; ++q) {
        const int64_t i = base + 4 * ((int64_t)q * kEwThreads + threadIdx.x);
        for (int e = 0; e < 4 && i + e < S.n; ++e) {
            const float g = Gt[i + e];
            float m = mb[i + e];
            if (S.carry) {
                m = ema(beta1, m, omb1, g);
                mb[i + e] = m;
            }
            float v = V[i + e], u;
            adam1(g, m, v, u, beta2, omb2, eps);
            V[i + e] = v;
            uo[i + e] = u;
        }
    }
}

// ------------------------------------------------ bf16-rotation variant ----

__device__ __forceinline__ int find_seg16(const Ew16Seg* segs, int nseg, int64_t chunk) {
    int lo = 0, hi = nseg - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (segs[mid].chunk_begin <= chunk) lo = mid; else hi = mid - 1;
    }
    return lo;
}

__device__ __forceinline__ u32x2 pack_bf16x4(f32x4 x) {
    u32x2 w;
    w.x = (uint32_t)f32_to_bf16(x[0]) | ((uint32_t)f32_to_bf16(x[1]) << 16);
    w.y = (uint32_t)f32_to_bf16(x[2]) | ((uint32_t)f32_to_bf16(x[3]) << 16);
    return w;
}

// UPDATE: the momentum update of momentum_kernel, plus bf16 copies of G (o1)
// and of the new M (o2, when set) for the rotations. Otherwise only the
// copies, of G and of M as stored.
template <bool UPDATE>
__global__ __launch_bounds__(kEwThreads) void momentum16_kernel(const Ew16Seg* __restrict__ segs, int nseg,
                                                                float beta1) {
    const int64_t chunk = blockIdx.x;
    const Ew16Seg S = segs[find_seg16(segs, nseg, chunk)];
    const int64_t base = (chunk - S.chunk_begin) * kEwChunk;
    const float omb = 1.f - beta1;
    if (S.vec && base + kEwChunk <= S.n) {
        f32x4 g[NQ], m[NQ];
        u32x2 raw[NQ];
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            const int64_t o = base + 4 * (q * kEwThreads + threadIdx.x);
            g[q] = *gptr((const f32x4*)(S.a + o));
            if (S.b_bf16) raw[q] = *gptr((const u32x2*)((const uint16_t*)S.b + o));
            else          m[q] = *gptr((const f32x4*)((const float*)S.b + o));
        }
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            const int64_t o = base + 4 * (q * kEwThreads + threadIdx.x);
            if (S.b_bf16) m[q] = widen_bf16x4(raw[q]);
            *gptr((u32x2*)(S.o1 + o)) = pack_bf16x4(g[q]);
            if (UPDATE) {
#pragma unroll
                for (int e = 0; e < 4; ++e) m[q][e] = ema(beta1, m[q][e], omb, g[q][e]);
                if (S.b_bf16) *gptr((u32x2*)((uint16_t*)S.b + o)) = pack_bf16x4(m[q]);
                else          *gptr((f32x4*)((float*)S.b + o)) = m[q];
            }
            if (S.o2) *gptr((u32x2*)(S.o2 + o)) = pack_bf16x4(m[q]);
        }
        return;
    }
    gmem<const float> G = gptr(S.a);
    for (int q = 0; q < NQ; ++q) {
        const int64_t i = base + 4 * ((int64_t)q * kEwThreads + threadIdx.x);
        for (int e = 0; e < 4 && i + e < S.n; ++e) {
            const float g = G[i + e];
            gptr(S.o1)[i + e] = f32_to_bf16(g);
            float mn;
            if (S.b_bf16) {
                gmem<uint16_t> p = gptr((uint16_t*)S.b + i + e);
                mn = bf16_to_f32(*p);
                if (UPDATE) {
                    mn = ema(beta1, mn, omb, g);
                    *p = f32_to_bf16(mn);
                }
            } else {
                gmem<float> p = gptr((float*)S.b + i + e);
                mn = *p;
                if (UPDATE) {
                    mn = ema(beta1, mn, omb, g);
                    *p = mn;
                }
            }
            if (S.o2) gptr(S.o2)[i + e] = f32_to_bf16(mn);
        }
    }
}

// v <- beta2 v + (1 - beta2) G~^2; u = m~ / (sqrt(v) + eps) stored as bf16 in
// o1. With carry, m~ (fp32, in b) is first advanced: b <- beta1 b + (1 - beta1) G~.
__global__ __launch_bounds__(kEwThreads) void adam16_kernel(const Ew16Seg* __restrict__ segs, int nseg,
                                                            float beta1, float beta2, float eps) {
    const int64_t chunk = blockIdx.x;
    const Ew16Seg S = segs[find_seg16(segs, nseg, chunk)];
    const int64_t base = (chunk - S.chunk_begin) * kEwChunk;
    const float omb1 = 1.f - beta1, omb2 = 1.f - beta2;
    if (S.vec && base + kEwChunk <= S.n) {
        f32x4 g[NQ], m[NQ], v[NQ];
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            const int64_t o = base + 4 * (q * kEwThreads + threadIdx.x);
            g[q] = *gptr((const f32x4*)(S.a + o));
            m[q] = *gptr((const f32x4*)((const float*)S.b + o));
            v[q] = *gptr((const f32x4*)(S.c + o));
        }
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            const int64_t o = base + 4 * (q * kEwThreads + threadIdx.x);
            f32x4 u;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                if (S.carry) m[q][e] = ema(beta1, m[q][e], omb1, g[q][e]);
                float ve = v[q][e], ue;
                adam1(g[q][e], m[q][e], ve, ue, beta2, omb2, eps);
                v[q][e] = ve;
                u[e] = ue;
            }
            *gptr((f32x4*)(S.c + o)) = v[q];
            if (S.carry) *gptr((f32x4*)((float*)S.b + o)) = m[q];
            *gptr((u32x2*)(S.o1 + o)) = pack_bf16x4(u);
        }
        return;
    }
    gmem<const float> Gt = gptr(S.a);
    gmem<float> mb = gptr((float*)S.b);
    gmem<float> V = gptr(S.c);
    for (int q = 0; q < NQ; ++q) {
        const int64_t i = base + 4 * ((int64_t)q * kEwThreads + threadIdx.x);
        for (int e = 0; e < 4 && i + e < S.n; ++e) {
            float m = mb[i + e];
            if (S.carry) {
                m = ema(beta1, m, omb1, Gt[i + e]);
                mb[i + e] = m;
            }
            float v = V[i + e], u;
            adam1(Gt[i + e], m, v, u, beta2, omb2, eps);
            V[i + e] = v;
            gptr(S.o1)[i + e] = f32_to_bf16(u);
        }
    }
}

// Element e of a job's padded destination: row e / ld_dst, column e % ld_dst.
__global__ __launch_bounds__(kEwThreads) void pack16_kernel(const PackJob* __restrict__ jobs, int njobs) {
    const int64_t chunk = blockIdx.x;
    int lo = 0, hi = njobs - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (jobs[mid].chunk_begin <= chunk) lo = mid; else hi = mid - 1;
    }
    const PackJob J = jobs[lo];
    const int64_t total = J.rows * J.ld_dst;
    const int64_t base = (chunk - J.chunk_begin) * kEwChunk;
    for (int k = threadIdx.x; k < kEwChunk; k += kEwThreads) {
        const int64_t e = base + k;
        if (e >= total) break;
        const int64_t r = e / J.ld_dst, c = e % J.ld_dst;
        uint16_t h = 0;
        if (c < J.cols) {
            const int64_t si = r * J.ld_src + c;
            h = J.src_bf16 ? gptr((const uint16_t*)J.src)[si] : f32_to_bf16(gptr((const float*)J.src)[si]);
        }
        gptr(J.dst)[e] = h;
    }
}

// One 32 x 32 tile of a basis: Xb[r][c] = X[r][c] and Xt[c][r] = X[r][c] for
// the tile's r, c < dp, with zeros where r or c >= d; rows of Xb and Xt past
// d are not stored. The transposed tile goes through LDS so that both the
// reads and the writes are along rows.
__global__ __launch_bounds__(256) void basis16_kernel(const BasisJob* __restrict__ jobs, int njobs) {
    __shared__ float tile[kBasisTile][kBasisTile + 1];
    const int bid = blockIdx.x;
    int lo = 0, hi = njobs - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (jobs[mid].tile_begin <= bid) lo = mid; else hi = mid - 1;
    }
    const BasisJob J = jobs[lo];
    const int per_row = (J.dp + kBasisTile - 1) / kBasisTile;
    const int t = bid - J.tile_begin;
    const int R = (t / per_row) * kBasisTile, Cc = (t % per_row) * kBasisTile;
    const int x = threadIdx.x & 31, y0 = threadIdx.x >> 5;
    for (int y = y0; y < kBasisTile; y += 8) {
        const int r = R + y, c = Cc + x;
        float val = 0.f;
        if (r < J.d && c < J.d)
            val = J.x_bf16 ? __uint_as_float((uint32_t)gptr((const uint16_t*)J.X)[(int64_t)r * J.d + c] << 16)
                           : gptr((const float*)J.X)[(int64_t)r * J.d + c];
        tile[y][x] = val;
        if (J.Xb && r < J.d && c < J.dp) gptr(J.Xb)[(int64_t)r * J.dp + c] = f32_to_bf16(val);
    }
    __syncthreads();
    for (int y = y0; y < kBasisTile; y += 8) {
        const int i = Cc + y, k = R + x;   // Xt[i][k] = X[k][i]
        if (i < J.d && k < J.dp) gptr(J.Xt)[(int64_t)i * J.dp + k] = f32_to_bf16(tile[x][y]);
    }
}

__global__ __launch_bounds__(kEwThreads) void cvt16_kernel(const CvtJob* __restrict__ jobs, int njobs) {
    const int64_t chunk = blockIdx.x;
    int lo = 0, hi = njobs - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (jobs[mid].chunk_begin <= chunk) lo = mid; else hi = mid - 1;
    }
    const CvtJob J = jobs[lo];
    const int64_t e0 = (chunk - J.chunk_begin) * kEwChunk;
    for (int64_t e = e0 + threadIdx.x; e < J.n && e < e0 + kEwChunk; e += kEwThreads) {
        if (J.to16) gptr((uint16_t*)J.dst)[e] = f32_to_bf16(gptr((const float*)J.src)[e]);
        else gptr((float*)J.dst)[e] = __uint_as_float((uint32_t)gptr((const uint16_t*)J.src)[e] << 16);
    }
}

__global__ __launch_bounds__(256) void transpose32_kernel(const TransposeJob* __restrict__ jobs, int njobs) {
    __shared__ float tile[kTransposeTile][kTransposeTile + 1];
    const int bid = blockIdx.x;
    int lo = 0, hi = njobs - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (jobs[mid].tile_begin <= bid) lo = mid; else hi = mid - 1;
    }
    const TransposeJob J = jobs[lo];
    const int per_row = (J.d + kTransposeTile - 1) / kTransposeTile;
    const int t = bid - J.tile_begin;
    const int R = (t / per_row) * kTransposeTile, Cc = (t % per_row) * kTransposeTile;
    const int x = threadIdx.x & 31, y0 = threadIdx.x >> 5;
    for (int y = y0; y < kTransposeTile; y += 8) {
        const int r = R + y, c = Cc + x;
        if (r < J.d && c < J.d) tile[y][x] = gptr(J.X)[(int64_t)r * J.d + c];
    }
    __syncthreads();
    for (int y = y0; y < kTransposeTile; y += 8) {
        const int i = Cc + y, k = R + x;   // Xt[i][k] = X[k][i]
        if (i < J.d && k < J.d) gptr(J.Xt)[(int64_t)i * J.d + k] = tile[x][y];
    }
}

// Tiles of a split job: tile t covers k in [32 (t / CT), +32), c in
// [32 (t % CT), +32) with CT = ceil(cols / 32) column tiles; the LDS tile is
// read along c and written along k.
__global__ __launch_bounds__(256) void split16_kernel(const SplitJob* __restrict__ jobs, int njobs) {
    __shared__ float tile[32][33];
    const int bid = blockIdx.x;
    int lo = 0, hi = njobs - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (jobs[mid].tile_begin <= bid) lo = mid; else hi = mid - 1;
    }
    const SplitJob J = jobs[lo];
    const int ct = (J.cols + 31) / 32;
    const int t = bid - J.tile_begin;
    const int k0 = (t / ct) * 32, c0 = (t % ct) * 32;
    const int x = threadIdx.x & 31, y0 = threadIdx.x >> 5;
    for (int y = y0; y < 32; y += 8) {
        const int k = k0 + y, c = c0 + x;
        float v = 0.f;
        if (k < J.rows && c < J.cols) {
            const int64_t si = (int64_t)k * J.ld_src + c;
            v = J.src_bf16 ? bf16_to_f32(gptr((const uint16_t*)J.src)[si]) : gptr((const float*)J.src)[si];
        }
        tile[y][x] = v;
    }
    __syncthreads();
    for (int y = y0; y < 32; y += 8) {
        const int c = c0 + y, k = k0 + x;
        if (c >= J.cols || k >= J.ld_dst) continue;
        const float v = tile[x][y];
        const int64_t di = (int64_t)c * J.ld_dst + k;
        const uint16_t h = f32_to_bf16(v);
        gptr(J.dst)[di] = h;
        if (J.npieces == 3) {
            const float r1 = v - bf16_to_f32(h);
            const uint16_t m = f32_to_bf16(r1);
            const float r2 = r1 - bf16_to_f32(m);
            gptr(J.dst)[J.piece_stride + di] = m;
            gptr(J.dst)[2 * J.piece_stride + di] = f32_to_bf16(r2);
        }
    }
}

}  // namespace

hipError_t launch_split16(const SplitJob* jobs, int njobs, int total_tiles, hipStream_t s) {
    if (njobs <= 0 || total_tiles <= 0) return hipSuccess;
    hipLaunchKernelGGL(split16_kernel, dim3((unsigned)total_tiles), dim3(256), 0, s, jobs, njobs);
    return hipGetLastError();
}

hipError_t launch_momentum16(const Ew16Seg* segs, int nseg, int64_t total_chunks, float beta1, hipStream_t s) {
    if (nseg <= 0 || total_chunks <= 0) return hipSuccess;
    hipLaunchKernelGGL(momentum16_kernel<true>, dim3((unsigned)total_chunks), dim3(kEwThreads), 0, s, segs, nseg,
                       beta1);
    return hipGetLastError();
}

hipError_t launch_convert16(const Ew16Seg* segs, int nseg, int64_t total_chunks, hipStream_t s) {
    if (nseg <= 0 || total_chunks <= 0) return hipSuccess;
    hipLaunchKernelGGL(momentum16_kernel<false>, dim3((unsigned)total_chunks), dim3(kEwThreads), 0, s, segs, nseg,
                       0.f);
    return hipGetLastError();
}

hipError_t launch_adam16(const Ew16Seg* segs, int nseg, int64_t total_chunks, float beta1, float beta2, float eps,
                         hipStream_t s) {
    if (nseg <= 0 || total_chunks <= 0) return hipSuccess;
    hipLaunchKernelGGL(adam16_kernel, dim3((unsigned)total_chunks), dim3(kEwThreads), 0, s, segs, nseg, beta1,
                       beta2, eps);
    return hipGetLastError();
}

hipError_t launch_pack16(const PackJob* jobs, int njobs, int64_t total_chunks, hipStream_t s) {
    if (njobs <= 0 || total_chunks <= 0) return hipSuccess;
    hipLaunchKernelGGL(pack16_kernel, dim3((unsigned)total_chunks), dim3(kEwThreads), 0, s, jobs, njobs);
    return hipGetLastError();
}

hipError_t launch_basis16(const BasisJob* jobs, int njobs, int total_tiles, hipStream_t s) {
    if (njobs <= 0 || total_tiles <= 0) return hipSuccess;
    hipLaunchKernelGGL(basis16_kernel, dim3((unsigned)total_tiles), dim3(256), 0, s, jobs, njobs);
    return hipGetLastError();
}

hipError_t launch_cvt16(const CvtJob* jobs, int njobs, int64_t total_chunks, hipStream_t s) {
    if (njobs <= 0 || total_chunks <= 0) return hipSuccess;
    hipLaunchKernelGGL(cvt16_kernel, dim3((unsigned)total_chunks), dim3(kEwThreads), 0, s, jobs, njobs);
    return hipGetLastError();
}

hipError_t launch_transpose32(const TransposeJob* jobs, int njobs, int total_tiles, hipStream_t s) {
    if (njobs <= 0 || total_tiles <= 0) return hipSuccess;
    hipLaunchKernelGGL(transpose32_kernel, dim3((unsigned)total_tiles), dim3(256), 0, s, jobs, njobs);
    return hipGetLastError();
}

hipError_t launch_momentum(const EwSeg* segs, int nseg, int64_t total_chunks, float beta1,
                           hipStream_t s) {
    if (nseg <= 0 || total_chunks <= 0) return hipSuccess;
    hipLaunchKernelGGL(momentum_kernel, dim3((unsigned)total_chunks), dim3(kEwThreads), 0, s, segs,
                       nseg, beta1);
    return hipGetLastError();
}

hipError_t launch_rotated_adam(const EwSeg* segs, int nseg, int64_t total_chunks, float beta1, float beta2,
                               float eps, hipStream_t s) {
    if (nseg <= 0 || total_chunks <= 0) return hipSuccess;
    hipLaunchKernelGGL(rotated_adam_kernel, dim3((unsigned)total_chunks), dim3(kEwThreads), 0, s,
                       segs, nseg, beta1, beta2, eps);
    return hipGetLastError();
}

}  // namespace matopt
