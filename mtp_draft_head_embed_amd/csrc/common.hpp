// common.hpp -- shared device helpers and the workspace layout of libmtpdraft.
//
// Internal to the library (not part of the C ABI).  gfx950 / CDNA4: wave64,
// 16-byte global loads, LDS for per-workgroup activations.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mtp {

constexpr int kWave = 64;

// ---------------------------------------------------------------------------
// Workspace layout (all offsets 256-byte aligned).
//   x        BF16 [B][H]        block input, written by the front half
//   partials (f32 value, u32 index) [B][kMaxHeadBlocks]  per-workgroup argmax
//   concat   BF16 [B][2H]       batched path: [enorm(e) | hnorm(h)]
//   xn       BF16 [B][H]        batched path: shared_head.norm(x)
//   P        FP32 [S][B][H]     batched path: eh_proj split-K partial sums
// ---------------------------------------------------------------------------
constexpr int kMaxHeadBlocks = 4096;
// Per sequence, the partial slots from kLogitSinkFirst on are never a
// workgroup's (the row kernels' grids stay below it): the single-sequence head
// stores each rounded logit into kLogitSinkSlots 2-byte slots there as it
// finishes the row (8 KiB, resident in L2), which keeps its rows streaming at
// full rate; the logits buffer is written from LDS in batches.
constexpr int kLogitSinkFirst = kMaxHeadBlocks / 2;
constexpr int kLogitSinkSlots = 4096;
static_assert(kLogitSinkSlots * 2 <= (kMaxHeadBlocks - kLogitSinkFirst) * 8,
              "the sink fits in the sequence's spare partial slots");

struct Partial {
    float val;
    uint32_t idx;
};

inline size_t align256(size_t n) { return (n + 255) & ~size_t(255); }

// The batched head deals its last tiles from kTilePools counters in the
// workspace, each on its own 4 KiB (so that they sit in different memory
// channels and their atomics do not queue behind one another).
constexpr int kTilePools = 8;
constexpr int kCtrStride = 4096;
// The single-sequence head deals its last passes of rows from kRowPools
// counters in the same slot (each taken far more often than a tile).
constexpr int kRowPools = 64;

struct WsLayout {
    size_t x_off, x_bytes;
    size_t part_off, part_bytes;
    size_t concat_off, xn_off, p_off;
    size_t ctr_off;  // the heads' counters, kCtrStride bytes apart (kTilePools or kRowPools of them)
    size_t total;
};

// eh_proj K-splits of the batched path for this hidden size (mfma_gemm.hip).
int eh_split_count(int hidden);

inline WsLayout ws_layout(int hidden, int batch)
{
    WsLayout L;
    const size_t bh = size_t(batch) * size_t(hidden);
    L.x_off = 0;
    L.x_bytes = align256(bh * 2);
    L.part_off = L.x_off + L.x_bytes;
    L.part_bytes = align256(size_t(batch) * kMaxHeadBlocks * sizeof(Partial));
    L.total = L.part_off + L.part_bytes;
    if (batch > 1) {
        L.concat_off = L.total;
        L.xn_off = L.concat_off + align256(bh * 4);
        L.p_off = L.xn_off + align256(bh * 2);
        L.total = L.p_off + align256(size_t(eh_split_count(hidden)) * bh * 4);
    } else {
        L.concat_off = L.xn_off = L.p_off = 0;
    }
    L.ctr_off = L.total;
    L.total += size_t(kRowPools > kTilePools ? kRowPools : kTilePools) * kCtrStride;
    return L;
}

// ---------------------------------------------------------------------------
// BF16 <-> f32
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t packed) { return __uint_as_float(packed << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t packed) { return __uint_as_float(packed & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

// Round to nearest even (finite inputs; NaN/Inf are outside the contract).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f)
{
    uint32_t u = __float_as_uint(f);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

// ---------------------------------------------------------------------------
// Wave reductions (fixed xor butterfly: the result does not depend on timing).
// ---------------------------------------------------------------------------
__device__ __forceinline__ float wave_sum(float v)
{
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1)
        v += __shfl_xor(v, m, kWave);
    return v;
}

__device__ __forceinline__ float wave_max(float v)
{
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1)
        v = fmaxf(v, __shfl_xor(v, m, kWave));
    return v;
}

// Argmax order: larger value first, then lower index.  Associative and
// commutative, so any reduction tree gives the same winner; -0 == +0.
__device__ __forceinline__ bool better(float v1, uint32_t i1, float v2, uint32_t i2)
{
    return (v1 > v2) || (v1 == v2 && i1 < i2);
}

__device__ __forceinline__ void wave_argmax(float &v, uint32_t &i)
{
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
        float ov = __shfl_xor(v, m, kWave);
        uint32_t oi = __shfl_xor(i, m, kWave);
        if (better(ov, oi, v, i)) {
            v = ov;
            i = oi;
        }
    }
}

// ---------------------------------------------------------------------------
// Vanilla RMSNorm pieces (x * w / sqrt(mean(x^2) + eps)) for one workgroup
// holding one BF16 vector; thread t owns elements (i*blockDim + t)*8 .. +8.
// The division by r is a multiplication by 1/r, correctly rounded once per
// vector: x * w is exact in FP32 (BF16 x BF16), so each output before its
// BF16 rounding is within about 31 units (2^-24) of the exact value (r itself
// within 30: the sum of squares rounds at most 54 times over positive terms,
// the square root halves that), against 30 with a division per element that
// costs ten instructions.
// ---------------------------------------------------------------------------
// Sum of squares of a BF16 vector of n elements (n % 8 == 0,
// n <= 4 * blockDim * 8), reduced over the whole workgroup in a fixed order.
// `v` receives the thread's 16-byte pieces (element (i*blockDim + tid)*8).
__device__ __forceinline__ float block_sumsq(const uint16_t *__restrict__ src, int n, bool valid,
                                             uint4 (&v)[4], float *red)
{
    const int tid = threadIdx.x;
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int j = (i * blockDim.x + tid) * 8;
        v[i] = make_uint4(0, 0, 0, 0);
        if (valid && j < n)
            v[i] = *reinterpret_cast<const uint4 *>(src + j);
        const uint32_t w[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float a = bf16_lo(w[q]), b = bf16_hi(w[q]);
            ss = fmaf(a, a, ss);
            ss = fmaf(b, b, ss);
        }
    }
    ss = wave_sum(ss);
    const int nw = blockDim.x / kWave;
    __syncthreads();
    if ((tid & (kWave - 1)) == 0)
        red[tid / kWave] = ss;
    __syncthreads();
    float tot = 0.f;
    for (int w = 0; w < nw; ++w)
        tot += red[w];
    return tot;
}

// out[j] = BF16(x_j * w_j / r) for the thread's pieces (dst in LDS or global).
__device__ __forceinline__ void norm_to_lds(const uint4 (&v)[4], const uint16_t *__restrict__ w,
                                            int n, float r, uint16_t *dst)
{
    const int tid = threadIdx.x;
    const float rr = 1.0f / r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int j = (i * blockDim.x + tid) * 8;
        if (j < n) {
            const uint4 wv = *reinterpret_cast<const uint4 *>(w + j);
            const uint32_t xa[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
            const uint32_t wa[4] = {wv.x, wv.y, wv.z, wv.w};
            uint32_t o[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float lo = (bf16_lo(xa[q]) * bf16_lo(wa[q])) * rr;
                const float hi = (bf16_hi(xa[q]) * bf16_hi(wa[q])) * rr;
                o[q] = pack_bf16x2(lo, hi);
            }
            *reinterpret_cast<uint4 *>(dst + j) = make_uint4(o[0], o[1], o[2], o[3]);
        }
    }
}

// The vanilla norms of the prologues, in two phases: *_load issues every
// load a thread needs (up to 4 x 8 elements of each vector, n <= 32
// blockDim.x), *_store reduces across the block and writes the normed BF16
// vector.  A kernel can issue its own first weight loads between the two:
// load completion is counted in issue order, so loads issued after the
// norm's do not hold up its reduction, while the reverse would.
__device__ __forceinline__ uint4 zero_unless(bool keep, const uint4 &v)
{
    return make_uint4(keep ? v.x : 0u, keep ? v.y : 0u, keep ? v.z : 0u, keep ? v.w : 0u);
}

struct DualNormIn {
    uint4 a[4], b[4], wa[4], wb[4];
};
struct SingleNormIn {
    uint4 a[4], wa[4];
};

// [norm(x0) with w0 | norm(x1) with w1], one block reduction for both
// (x0 reads as zeros when !valid0).
__device__ __forceinline__ DualNormIn dual_norm_load(const uint16_t *__restrict__ x0, bool valid0,
                                                     const uint16_t *__restrict__ w0,
                                                     const uint16_t *__restrict__ x1,
                                                     const uint16_t *__restrict__ w1, int n)
{
    const int tid = threadIdx.x;
    DualNormIn v;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int j = (i * blockDim.x + tid) * 8;
        // load from a clamped index and select, rather than branch around
        // the load (which would blur the wait counts of the loads after it)
        const bool in = j < n;
        const int jc = in ? j : 0;
        v.a[i] = zero_unless(in && valid0, *reinterpret_cast<const uint4 *>(x0 + jc));
        v.b[i] = zero_unless(in, *reinterpret_cast<const uint4 *>(x1 + jc));
        v.wa[i] = zero_unless(in, *reinterpret_cast<const uint4 *>(w0 + jc));
        v.wb[i] = zero_unless(in, *reinterpret_cast<const uint4 *>(w1 + jc));
    }
    return v;
}

__device__ __forceinline__ void dual_norm_store(const DualNormIn &v, int n, float eps,
                                                uint16_t *dst0, uint16_t *dst1, float *red)
{
    const int tid = threadIdx.x;
    float s0 = 0.f, s1 = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t pa[4] = {v.a[i].x, v.a[i].y, v.a[i].z, v.a[i].w};
        const uint32_t pb[4] = {v.b[i].x, v.b[i].y, v.b[i].z, v.b[i].w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            s0 = fmaf(bf16_lo(pa[q]), bf16_lo(pa[q]), s0);
            s0 = fmaf(bf16_hi(pa[q]), bf16_hi(pa[q]), s0);
            s1 = fmaf(bf16_lo(pb[q]), bf16_lo(pb[q]), s1);
            s1 = fmaf(bf16_hi(pb[q]), bf16_hi(pb[q]), s1);
        }
    }
    s0 = wave_sum(s0);
    s1 = wave_sum(s1);
    const int nw = blockDim.x / kWave;
    __syncthreads();
    if ((tid & (kWave - 1)) == 0) {
        red[tid / kWave] = s0;
        red[16 + tid / kWave] = s1;
    }
    __syncthreads();
    float t0 = 0.f, t1 = 0.f;
    for (int w = 0; w < nw; ++w) {
        t0 += red[w];
        t1 += red[16 + w];
    }
    const float rr0 = 1.0f / sqrtf(t0 / float(n) + eps);
    const float rr1 = 1.0f / sqrtf(t1 / float(n) + eps);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int j = (i * blockDim.x + tid) * 8;
        if (j < n) {
            const uint32_t pa[4] = {v.a[i].x, v.a[i].y, v.a[i].z, v.a[i].w};
            const uint32_t pb[4] = {v.b[i].x, v.b[i].y, v.b[i].z, v.b[i].w};
            const uint32_t qa[4] = {v.wa[i].x, v.wa[i].y, v.wa[i].z, v.wa[i].w};
            const uint32_t qb[4] = {v.wb[i].x, v.wb[i].y, v.wb[i].z, v.wb[i].w};
            uint32_t oa[4], ob[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                oa[q] = pack_bf16x2((bf16_lo(pa[q]) * bf16_lo(qa[q])) * rr0,
                                    (bf16_hi(pa[q]) * bf16_hi(qa[q])) * rr0);
                ob[q] = pack_bf16x2((bf16_lo(pb[q]) * bf16_lo(qb[q])) * rr1,
                                    (bf16_hi(pb[q]) * bf16_hi(qb[q])) * rr1);
            }
            *reinterpret_cast<uint4 *>(dst0 + j) = make_uint4(oa[0], oa[1], oa[2], oa[3]);
            *reinterpret_cast<uint4 *>(dst1 + j) = make_uint4(ob[0], ob[1], ob[2], ob[3]);
        }
    }
}

__device__ __forceinline__ void dual_norm(const uint16_t *__restrict__ x0, bool valid0,
                                          const uint16_t *__restrict__ w0,
                                          const uint16_t *__restrict__ x1,
                                          const uint16_t *__restrict__ w1, int n, float eps,
                                          uint16_t *dst0, uint16_t *dst1, float *red)
{
    dual_norm_store(dual_norm_load(x0, valid0, w0, x1, w1, n), n, eps, dst0, dst1, red);
}

// One vanilla norm with the vector and its weight loaded together.
__device__ __forceinline__ SingleNormIn single_norm_load(const uint16_t *__restrict__ x,
                                                         const uint16_t *__restrict__ w, int n)
{
    const int tid = threadIdx.x;
    SingleNormIn v;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int j = (i * blockDim.x + tid) * 8;
        const bool in = j < n;
        const int jc = in ? j : 0;
        v.a[i] = zero_unless(in, *reinterpret_cast<const uint4 *>(x + jc));
        v.wa[i] = zero_unless(in, *reinterpret_cast<const uint4 *>(w + jc));
    }
    return v;
}

__device__ __forceinline__ void single_norm_store(const SingleNormIn &v, int n, float eps,
                                                  uint16_t *dst, float *red)
{
    const int tid = threadIdx.x;
    float s0 = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t pa[4] = {v.a[i].x, v.a[i].y, v.a[i].z, v.a[i].w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            s0 = fmaf(bf16_lo(pa[q]), bf16_lo(pa[q]), s0);
            s0 = fmaf(bf16_hi(pa[q]), bf16_hi(pa[q]), s0);
        }
    }
    s0 = wave_sum(s0);
    const int nw = blockDim.x / kWave;
    __syncthreads();
    if ((tid & (kWave - 1)) == 0)
        red[tid / kWave] = s0;
    __syncthreads();
    float t0 = 0.f;
    for (int w2 = 0; w2 < nw; ++w2)
        t0 += red[w2];
    const float rr0 = 1.0f / sqrtf(t0 / float(n) + eps);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int j = (i * blockDim.x + tid) * 8;
        if (j < n) {
            const uint32_t pa[4] = {v.a[i].x, v.a[i].y, v.a[i].z, v.a[i].w};
            const uint32_t qa[4] = {v.wa[i].x, v.wa[i].y, v.wa[i].z, v.wa[i].w};
            uint32_t oa[4];
#pragma unroll
            for (int q = 0; q < 4; ++q)
                oa[q] = pack_bf16x2((bf16_lo(pa[q]) * bf16_lo(qa[q])) * rr0,
                                    (bf16_hi(pa[q]) * bf16_hi(qa[q])) * rr0);
            *reinterpret_cast<uint4 *>(dst + j) = make_uint4(oa[0], oa[1], oa[2], oa[3]);
        }
    }
}

__device__ __forceinline__ void single_norm(const uint16_t *__restrict__ x,
                                            const uint16_t *__restrict__ w, int n, float eps,
                                            uint16_t *dst, float *red)
{
    single_norm_store(single_norm_load(x, w, n), n, eps, dst, red);
}

}  // namespace mtp
