// Grouped bf16 MFMA GEMM for gfx950 (CDNA4): C = alpha A B^T (+ beta C).
//
// Serves the four rotations of the bf16-rotation variant. Every product is
// arranged so that both operands are stored with k contiguous (A is M x K,
// B is N x K, both row-major): with a bf16 operand each lane of
// v_mfma_f32_32x32x16_bf16 takes eight consecutive k values of one row, one
// 16-byte LDS read, and an operand whose k index is strided would need a
// transposing stage instead.
//
// Tiles. Cfg16<WAVES_M, WAVES_N, BLK_M, BLK_N>: each wavefront holds a
// (32 BLK_M) x (32 BLK_N) block of the output as BLK_M x BLK_N accumulators
// of 32 x 32. The large configuration is a 256 x 256 tile of 8 wavefronts
// (2 x 4) of 128 x 64: per 16-deep k step a wavefront reads 4 + 2 fragments
// (6 KiB of LDS) for 8 MFMAs, and with two wavefronts per SIMD one's LDS
// reads, waits and barrier are covered by the other's MFMAs (measured 10 %
// faster on the pieced momentum products than 4 wavefronts of 128 x 128,
// one per SIMD, which read half as much LDS per MFMA). K advances in slabs
// of 64 (128 bytes per row) through two LDS buffers.
//
// Staging. Operands go from global memory straight into LDS
// (global_load_lds, 16 bytes per lane: one wavefront instruction writes 8
// rows of 128 bytes). The 16-byte group q of row r lands in slot
// q ^ ((r ^ r/8) mod 8): the 16 lanes of one read phase (rows r..r+15, one
// group) then hit distinct bank groups for both 32- and 64-bank LDS. Loads
// outside the operand (rows past M or N, k past K) read a zero block instead,
// so padded slots add nothing and no k tail needs clearing.
//
// Pipeline (as in the fp32 GEMM): the fill of slab k+1 is issued before the
// MFMAs of slab k; the fragments of k step s+1 are read after the first row
// of MFMAs of step s; the slab barrier sits before the last step's MFMAs.
//
// Work distribution: one workgroup per output tile, problems concatenated in
// tile space in longest-processing-time order by the host, workgroup ids
// remapped so that each XCD gets runs of neighbouring tiles.
#include "variant_bf16.h"

namespace matopt {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Zero bytes read by every load that falls outside an operand.
__device__ __attribute__((aligned(64))) uint32_t g_gemm16_zero[16];

namespace {

#ifndef MATOPT_GEMM16_XCD_RUN
#define MATOPT_GEMM16_XCD_RUN 16
#endif
#ifndef MATOPT_GEMM16_GROUP_M
#define MATOPT_GEMM16_GROUP_M 4
#endif
constexpr int XCD = 8;
constexpr int XCD_RUN = MATOPT_GEMM16_XCD_RUN;
constexpr int GROUP_M = MATOPT_GEMM16_GROUP_M;

// SLAB_K: k values per LDS slab (rows of 2 SLAB_K bytes); STAGES: LDS
// buffers in the fill ring (2: fill slab k+1 during slab k; 4: slab k+3).
template <int WAVES_M, int WAVES_N, int BLK_M, int BLK_N, int SLAB_K = 64, int STAGES = 2>
struct Cfg16 {
    static constexpr int WM = WAVES_M, WN = WAVES_N, TM = BLK_M, TN = BLK_N;
    static constexpr int BK = SLAB_K, ST = STAGES;
    static constexpr int RB = 2 * BK;      // bytes per LDS row
    static constexpr int CH = BK / 8;      // 16-byte groups per row
    static constexpr int NS = BK / 16;     // MFMA k steps per slab
    static constexpr int NT = 64 * WM * WN, NW = NT / 64;
    static constexpr int BM = 32 * TM * WM, BN = 32 * TN * WN;
    static constexpr int AB = BM * RB, BB = BN * RB;   // bytes of one A / B buffer
    static constexpr int SMEM = ST * (AB + BB);
    static constexpr int DMA_PER_SLAB = (AB + BB) / 1024 / NW;   // fill instructions per wavefront
    static_assert(BK == 32 || BK == 64, "slabs of 32 or 64 k values");
    static_assert(ST == 2 || ST == 4, "two or four LDS stages");
    static_assert((AB / 1024) % NW == 0 && (BB / 1024) % NW == 0, "tile not divisible into LDS chunks");
    static_assert(ST == 4 || NS % 2 == 0, "the last k step's fragments are in slot 1");
};
#ifndef MATOPT_GEMM16_LARGE
#define MATOPT_GEMM16_LARGE 2, 4, 4, 2, 64, 2
#endif
using Small16 = Cfg16<2, 2, 2, 2>;
using Large16 = Cfg16<MATOPT_GEMM16_LARGE>;
static_assert(Small16::BM == kGemm16Cfgs[0].bm && Small16::BN == kGemm16Cfgs[0].bn, "tile size mismatch");
static_assert(Large16::BM == kGemm16Cfgs[1].bm && Large16::BN == kGemm16Cfgs[1].bn, "tile size mismatch");

// Slot of 16-byte group q of LDS row r: q ^ swz16<BK>(r). With 8 groups per
// row (r ^ r/8) mod 8, with 4 groups ((r/2) ^ (r/4)) mod 4: the 16 lanes of a
// read phase (rows r..r+15 of one group) hit distinct bank groups for both
// 32- and 64-bank LDS.
template <int BK>
__device__ __forceinline__ int swz16(int r) {
    if constexpr (BK == 64) return (r ^ (r >> 3)) & 7;
    else return ((r >> 1) ^ (r >> 2)) & 3;
}

typedef __attribute__((address_space(3))) void* lds_ptr;
typedef __attribute__((address_space(1))) const void* gsrc_ptr;

// One slab (R rows x BK k) of an operand into LDS buffer `buf`: rows r0.. of
// a row-major bf16 matrix with `rows` rows, k0.. of its K columns.
template <class C, int R>
__device__ __forceinline__ void dma16(char* buf, const uint16_t* base, int64_t ld, int rows, int K, int r0,
                                      int k0) {
    constexpr int RPC = 1024 / C::RB;    // rows per 1 KiB chunk
    constexpr int CPW = R / RPC / C::NW; // chunks per wavefront
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
#pragma unroll
    for (int t = 0; t < CPW; ++t) {
        const int c = wave * CPW + t;
        const int r = RPC * c + lane / C::CH;
        const int k = k0 + 8 * ((lane % C::CH) ^ swz16<C::BK>(r));
        const int grow = r0 + r;
        const void* src = (grow < rows && k < K) ? (const void*)(base + (int64_t)grow * ld + k)
                                                  : (const void*)g_gemm16_zero;
        __builtin_amdgcn_global_load_lds((gsrc_ptr)src, (lds_ptr)(buf + c * 1024), 16, 0, 0);
    }
}

// The same fill with the per-lane addresses computed once per tile: each
// chunk's byte offset from the operand's slab-0 origin (row clamped into the
// operand, 32-bit: the caller checks the operand's span) and whether its row
// is inside the operand. A slab whose k values all lie inside K then loads
// from origin + k0 (uniform) plus the offset, or the zero block for rows
// past the operand.
template <class C, int R>
struct Dma16Offs {
    static constexpr int RPC = 1024 / C::RB;
    static constexpr int CPW = R / RPC / C::NW;
    uint32_t off[CPW];
    uint32_t rok;   // bit t: chunk t's row is inside the operand

    __device__ __forceinline__ void init(int64_t ld, int rows, int r0) {
        const int lane = threadIdx.x & 63;
        const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
        rok = 0;
#pragma unroll
        for (int t = 0; t < CPW; ++t) {
            const int c = wave * CPW + t;
            const int r = RPC * c + lane / C::CH;
            const int kp = 8 * ((lane % C::CH) ^ swz16<C::BK>(r));
            const int grow = r0 + r;
            const int rc = grow < rows ? grow : rows - 1;
            off[t] = (uint32_t)(((int64_t)rc * ld + kp) * 2);
            rok |= (grow < rows ? 1u : 0u) << t;
        }
    }

    __device__ __forceinline__ void fill(char* buf, const uint16_t* base, int k0) const {
        const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
        const char* origin = (const char*)(base + k0);
#pragma unroll
        for (int t = 0; t < CPW; ++t) {
            const int c = wave * CPW + t;
            const void* src = ((rok >> t) & 1u) ? (const void*)(origin + off[t]) : (const void*)g_gemm16_zero;
            __builtin_amdgcn_global_load_lds((gsrc_ptr)src, (lds_ptr)(buf + c * 1024), 16, 0, 0);
        }
    }
};

// Fragments of k step s: lane l takes row (or column) l % 32 of each 32-block
// and k values 16 s + 8 (l / 32) .. +7 of the slab.
template <class C>
__device__ __forceinline__ void frags16(const char* As, const char* Bs, int s, int wm, int wn, int lane,
                                        bf16x8 (&a)[C::TM], bf16x8 (&b)[C::TN]) {
    const int q = 2 * s + (lane >> 5), l32 = lane & 31;
#pragma unroll
    for (int i = 0; i < C::TM; ++i) {
        const int row = wm * 32 * C::TM + i * 32 + l32;
        a[i] = *(const bf16x8*)(As + row * C::RB + ((q ^ swz16<C::BK>(row)) << 4));
    }
#pragma unroll
    for (int j = 0; j < C::TN; ++j) {
        const int col = wn * 32 * C::TN + j * 32 + l32;
        b[j] = *(const bf16x8*)(Bs + col * C::RB + ((q ^ swz16<C::BK>(col)) << 4));
    }
}

// MFMAs of accumulator rows I0 .. I1-1 for one k step.
template <class C, int I0, int I1>
__device__ __forceinline__ void mma16(const bf16x8 (&a)[C::TM], const bf16x8 (&b)[C::TN],
                                      f32x16 (&acc)[C::TM][C::TN]) {
#pragma unroll
    for (int i = I0; i < I1; ++i)
#pragma unroll
        for (int j = 0; j < C::TN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
}

__device__ __forceinline__ uint16_t to_bf16(float x) {
    return __builtin_bit_cast(uint16_t, (__bf16)x);
}

// Epilogue through LDS. Accumulator register r of lane l holds row
// 8 (r / 4) + 4 (l / 32) + r % 4, column l % 32 of its 32 x 32 block, so a
// direct store would write four rows per register group with 4-byte accesses.
// Instead each wavefront copies one 32-row slice of its block (32 x 32 TN
// values) into its own LDS region, row-major with a row stride of
// 32 TN + 8 floats (the two half-waves, 4 rows apart, then fill all 64 banks),
// reads it back as 16-byte row segments and writes those with 16-byte stores
// (8-byte for bf16), reading old C the same way when beta != 0. The LDS
// buffers are free once every wavefront has passed the barrier that follows
// the main loop.
template <class C>
struct Epi16 {
    static constexpr int W = 32 * C::TN;        // columns of a wavefront's block
    static constexpr int LD = W + 8;            // LDS row stride (floats)
    static constexpr int REGION = 32 * LD;      // floats per wavefront
    static constexpr int LPR = W / 4;           // lanes per row (4 floats each)
    static constexpr int RPI = 64 / LPR;        // rows per read instruction
    static_assert(C::NW * REGION * 4 <= C::SMEM, "epilogue staging does not fit in LDS");
    static_assert(64 % LPR == 0, "a row must split evenly over the lanes");
};

template <class C, bool OUT16>
__device__ __forceinline__ void epi16(const Gemm16Prob& p, int m0, int n0, int wm, int wn, int lane,
                                      const f32x16 (&acc)[C::TM][C::TN], float alpha, char* smem) {
    using E = Epi16<C>;
    const int h = lane >> 5, l32 = lane & 31;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    float* reg = (float*)smem + wave * E::REGION;
    const int col0 = n0 + wn * E::W;
    // 16-byte (fp32) or 8-byte (bf16) groups of 4 columns need ldc % 4 == 0 and an aligned C
    const bool vec = (p.ldc % 4 == 0) && (((uintptr_t)p.C) % (OUT16 ? 8 : 16) == 0);
    const int lim = OUT16 ? p.pad_n : p.N;   // columns stored (bf16: zeros in [N, pad_n))
    __syncthreads();
#pragma unroll
    for (int i = 0; i < C::TM; ++i) {
#pragma unroll
        for (int j = 0; j < C::TN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                reg[(8 * (r >> 2) + 4 * h + (r & 3)) * E::LD + j * 32 + l32] = alpha * acc[i][j][r];
        __syncthreads();
        const int row0 = m0 + wm * 32 * C::TM + i * 32;
#pragma unroll
        for (int it = 0; it < 32 / E::RPI; ++it) {
            const int rl = it * E::RPI + lane / E::LPR, c4 = 4 * (lane % E::LPR);
            const int row = row0 + rl, col = col0 + c4;
            const f32x4 v = *(const f32x4*)&reg[rl * E::LD + c4];
            if (row >= p.M || col >= lim) continue;
            const int64_t off = (int64_t)row * p.ldc + col;
            if (OUT16) {
                uint16_t o[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) o[e] = col + e < p.N ? to_bf16(v[e]) : 0;
                if (vec && col + 3 < lim) {
                    u32x2 w;
                    w.x = (uint32_t)o[0] | ((uint32_t)o[1] << 16);
                    w.y = (uint32_t)o[2] | ((uint32_t)o[3] << 16);
                    *gptr((u32x2*)((uint16_t*)p.C + off)) = w;
                } else {
                    for (int e = 0; e < 4 && col + e < lim; ++e) gptr((uint16_t*)p.C)[off + e] = o[e];
                }
            } else {
                f32x4 out = v;
                if (vec && col + 3 < lim) {
                    if (p.beta != 0.f) {
                        const f32x4 old = *gptr((const f32x4*)((const float*)p.C + off));
#pragma unroll
                        for (int e = 0; e < 4; ++e) out[e] += p.beta * old[e];
                    }
                    *gptr((f32x4*)((float*)p.C + off)) = out;
                } else {
                    for (int e = 0; e < 4 && col + e < lim; ++e) {
                        float x = out[e];
                        if (p.beta != 0.f) x += p.beta * gptr((const float*)p.C)[off + e];
                        gptr((float*)p.C)[off + e] = x;
                    }
                }
            }
        }
        __syncthreads();
    }
}

// s_waitcnt immediate (gfx9 layout) that waits until at most `vm` vector
// memory operations of this wavefront are outstanding (and, with lgkm0, all
// LDS reads have returned); the other counters are left alone.
constexpr int waitcnt_imm(int vm, bool lgkm0) {
    return (vm & 15) | (7 << 4) | ((lgkm0 ? 0 : 15) << 8) | ((vm >> 4) << 14);
}

// Slab barrier. With two stages the next slab's fill is the only one in
// flight and __syncthreads (which drains every counter) is exact. With a
// ring of ST stages each wavefront waits only until the fill of the next
// slab has landed, leaving the ST - 2 newer fills in flight (fills complete
// in issue order), and until its own LDS reads of the slab being released
// have returned; the barrier then makes every wavefront's part visible. The
// empty asm statements keep the compiler from moving memory accesses across.
template <class C>
__device__ __forceinline__ void slab_barrier() {
    if constexpr (C::ST == 2) {
        __syncthreads();
    } else {
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_waitcnt(waitcnt_imm((C::ST - 2) * C::DMA_PER_SLAB, true));
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    }
}

template <class C, bool OUT16>
__device__ __forceinline__ void tile16(const Gemm16Prob& p, int tm, int tn, float alpha_scale, char* smem) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave % C::WM, wn = wave / C::WM;
    const int m0 = tm * C::BM, n0 = tn * C::BN;
    // ring buffer b of A at smem + b AB, of B at smem + ST AB + b BB
    auto abuf = [&](int b) { return smem + b * C::AB; };
    auto bbuf = [&](int b) { return smem + C::ST * C::AB + b * C::BB; };
    // Pieced products with two stages run their slabs k-slab by k-slab, the
    // periods of one k-slab back to back: slab t is k-slab t / np of period
    // t % np. An operand read again in every period (piece stride 0) is then
    // filled once per k-slab and stays in its buffer (k-slab parity) while
    // the other operand's pieces stream through theirs (slab parity), so
    // the fills move (np + 1) instead of 2 np operand slabs per k-slab.
    const bool inter = C::ST == 2 && p.np > 1;
    auto buf_a = [&](int t) { return inter && p.a_ps == 0 ? (t / p.np) & 1 : t & 1; };
    auto buf_b = [&](int t) { return inter && p.b_ps == 0 ? (t / p.np) & 1 : t & 1; };
    // Otherwise slab t covers k0 = t BK of the concatenated range: period q
    // at kk = k0 - q kper (kper is a multiple of the slab depth). Past the
    // last slab every load reads the zero block.
    // per-tile fill addresses, when both operands' spans fit 32-bit offsets
    Dma16Offs<C, C::BM> oa;
    Dma16Offs<C, C::BN> ob;
    const bool offs = (int64_t)p.M * p.lda * 2 < (int64_t(1) << 32) && (int64_t)p.N * p.ldb * 2 < (int64_t(1) << 32);
    if (offs) {
        oa.init(p.lda, p.M, m0);
        ob.init(p.ldb, p.N, n0);
    }
    // slab of k values k0 .. k0 + BK - 1 of period q, inside K or not (kv = 0:
    // past the last slab)
    auto fill_a = [&](char* buf, int q, int kv, int k0) {
        if (offs && kv > 0 && k0 + C::BK <= kv) oa.fill(buf, p.A + q * p.a_ps, k0);
        else dma16<C, C::BM>(buf, p.A + q * p.a_ps, p.lda, p.M, kv, m0, k0);
    };
    auto fill_b = [&](char* buf, int q, int kv, int k0) {
        if (offs && kv > 0 && k0 + C::BK <= kv) ob.fill(buf, p.B + q * p.b_ps, k0);
        else dma16<C, C::BN>(buf, p.B + q * p.b_ps, p.ldb, p.N, kv, n0, k0);
    };
    auto fill = [&](int b, int t) {
        if (inter) {
            const int ks = t / p.np, q = t - ks * p.np;
            const int k0 = ks * C::BK;
            const int kv = k0 < p.K ? p.K : 0;
            if (p.a_ps != 0 || q == 0) fill_a(abuf(buf_a(t)), q, kv, k0);
            if (p.b_ps != 0 || q == 0) fill_b(bbuf(buf_b(t)), q, kv, k0);
            return;
        }
        const int k0 = t * C::BK;
        int q = k0 / p.kper;
        const int kk = k0 - q * p.kper;
        const int kv = q < p.np ? p.K : 0;
        q = min(q, p.np - 1);
        fill_a(abuf(b), q, kv, kk);
        fill_b(bbuf(b), q, kv, kk);
    };
    f32x16 acc[C::TM][C::TN];
#pragma unroll
    for (int i = 0; i < C::TM; ++i)
#pragma unroll
        for (int j = 0; j < C::TN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
    const int nk = p.np == 1 ? (p.K + C::BK - 1) / C::BK
                 : inter    ? p.np * ((p.K + C::BK - 1) / C::BK)
                            : p.np * (p.kper / C::BK);
    const float alpha = p.alpha * alpha_scale;
    if (nk == 0) {
        epi16<C, OUT16>(p, m0, n0, wm, wn, lane, acc, alpha, smem);
        return;
    }
    // slabs 0 .. ST-2 in flight; slab 0 landed before the first reads
#pragma unroll
    for (int st = 0; st < C::ST - 1; ++st) fill(st, st);
    slab_barrier<C>();
    bf16x8 fa[2][C::TM], fb[2][C::TN];
    frags16<C>(abuf(0), bbuf(0), 0, wm, wn, lane, fa[0], fb[0]);
    int cur = 0;
    for (int kt = 0; kt < nk; ++kt) {
        const int nxt = cur + 1 == C::ST ? 0 : cur + 1;
        const int fb_ = cur == 0 ? C::ST - 1 : cur - 1;   // buffer of slab kt + ST - 1
        const char* As = abuf(inter ? buf_a(kt) : cur);
        const char* Bs = bbuf(inter ? buf_b(kt) : cur);
        // past the last slab the fill reads only the zero block into an idle buffer
        fill(fb_, kt + C::ST - 1);
#pragma unroll
        for (int s = 0; s < C::NS - 1; ++s) {
            mma16<C, 0, 1>(fa[s & 1], fb[s & 1], acc);
            __builtin_amdgcn_sched_barrier(0);
            frags16<C>(As, Bs, s + 1, wm, wn, lane, fa[(s + 1) & 1], fb[(s + 1) & 1]);
            __builtin_amdgcn_sched_barrier(0);
            mma16<C, 1, C::TM>(fa[s & 1], fb[s & 1], acc);
            __builtin_amdgcn_sched_barrier(0);
        }
        slab_barrier<C>();
        mma16<C, 0, 1>(fa[1], fb[1], acc);
        __builtin_amdgcn_sched_barrier(0);
        frags16<C>(abuf(inter ? buf_a(kt + 1) : nxt), bbuf(inter ? buf_b(kt + 1) : nxt), 0, wm, wn, lane, fa[0],
                   fb[0]);
        __builtin_amdgcn_sched_barrier(0);
        mma16<C, 1, C::TM>(fa[1], fb[1], acc);
        __builtin_amdgcn_sched_barrier(0);
        cur = nxt;
    }
    epi16<C, OUT16>(p, m0, n0, wm, wn, lane, acc, alpha, smem);
}

// Tile -> (row, column) of tiles, grouped by GROUP_M tile rows for L2 reuse.
__device__ __forceinline__ void raster16(int t, int tiles_m, int tiles_n, int& tm, int& tn) {
    const int per_group = GROUP_M * tiles_n;
    const int gidx = t / per_group;
    const int first = gidx * GROUP_M;
    const int gsz = min(tiles_m - first, GROUP_M);
    const int r = t - gidx * per_group;
    tm = first + r % gsz;
    tn = r / gsz;
}

// Workgroup id -> logical tile: within each full window of XCD * XCD_RUN
// ids, the ids the dispatcher sends to one XCD get XCD_RUN consecutive tiles.
__device__ __forceinline__ int xcd_remap16(int bid, int total) {
    const int win = XCD * XCD_RUN;
    const int w0 = (bid / win) * win;
    if (w0 + win > total) return bid;
    const int r = bid - w0;
    return w0 + (r % XCD) * XCD_RUN + r / XCD;
}

struct Gemm16Args {
    const Gemm16Prob* probs;
    const int32_t* tile_begin;
    int nprob;
    int total_tiles;
    float alpha_scale;
    Gemm16Prob single;
};

template <class C, bool OUT16>
__global__ __launch_bounds__(C::NT) void gemm16_kernel(Gemm16Args args) {
    __shared__ __attribute__((aligned(16))) char smem[C::SMEM];
    const int bid = xcd_remap16(blockIdx.x, args.total_tiles);
    Gemm16Prob p;
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
    raster16(t, p.tiles_m, p.tiles_n, tm, tn);
    tile16<C, OUT16>(p, tm, tn, args.alpha_scale, smem);
}

template <bool OUT16>
hipError_t launch16(int cfg, const Gemm16Args& a, hipStream_t s) {
    if (a.total_tiles <= 0) return hipSuccess;
    if (cfg == 1)
        gemm16_kernel<Large16, OUT16><<<dim3(a.total_tiles), dim3(Large16::NT), 0, s>>>(a);
    else
        gemm16_kernel<Small16, OUT16><<<dim3(a.total_tiles), dim3(Small16::NT), 0, s>>>(a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm16_grouped(bool c_bf16, int cfg, const Gemm16Prob* probs, const int32_t* tile_begin,
                                 int nprob, int total_tiles, float alpha_scale, hipStream_t s) {
    if (nprob <= 0) return hipSuccess;
    Gemm16Args a{};
    a.probs = probs;
    a.tile_begin = tile_begin;
    a.nprob = nprob;
    a.total_tiles = total_tiles;
    a.alpha_scale = alpha_scale;
    return c_bf16 ? launch16<true>(cfg, a, s) : launch16<false>(cfg, a, s);
}

hipError_t launch_gemm16_single(bool c_bf16, int cfg, const Gemm16Prob& prob, hipStream_t s) {
    Gemm16Args a{};
    a.nprob = 0;
    a.total_tiles = prob.tiles_m * prob.tiles_n;
    a.alpha_scale = 1.f;
    a.single = prob;
    return c_bf16 ? launch16<true>(cfg, a, s) : launch16<false>(cfg, a, s);
}

}  // namespace matopt
