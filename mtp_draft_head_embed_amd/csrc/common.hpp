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
// ---------------------------------------------------------------------------
constexpr int kMaxHeadBlocks = 4096;

struct Partial {
    float val;
    uint32_t idx;
};

inline size_t align256(size_t n) { return (n + 255) & ~size_t(255); }

struct WsLayout {
    size_t x_off, x_bytes;
    size_t part_off, part_bytes;
    size_t total;
};

inline WsLayout ws_layout(int hidden, int batch)
{
    WsLayout L;
    L.x_off = 0;
    L.x_bytes = align256(size_t(batch) * size_t(hidden) * 2);
    L.part_off = L.x_off + L.x_bytes;
    L.part_bytes = align256(size_t(batch) * kMaxHeadBlocks * sizeof(Partial));
    L.total = L.part_off + L.part_bytes;
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

}  // namespace mtp
