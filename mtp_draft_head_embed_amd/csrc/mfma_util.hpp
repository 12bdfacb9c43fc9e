// mfma_util.hpp -- operand helpers shared by the matrix-core kernels of the
// batched sweep (mfma_gemm.hip, tile_gemm.hip).  Internal to the library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mtp {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 ld_nt16(const char *p)
{
    const u32x4v v = __builtin_nontemporal_load(reinterpret_cast<const u32x4v *>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

// 16-byte buffer load with the non-temporal hint; offsets outside the
// resource's range return zero.
__device__ __forceinline__ uint4 ld_buf16(__amdgpu_buffer_rsrc_t r, int off)
{
    const u32x4v v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 2);
    return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ bf16x8 as_bf16x8(const uint4 &u)
{
    bf16x8 r;
    __builtin_memcpy(&r, &u, 16);
    return r;
}

// 8 E4M3FN codes (two dwords) -> 8 BF16 values, in order (scale 1: exact
// for every E4M3FN value).
__device__ __forceinline__ bf16x8 fp8x8_to_bf16(uint32_t lo, uint32_t hi)
{
    const bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
    const bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
    const bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
    const bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
    bf16x8 r;
    r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
    r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
    return r;
}

// The buffer-resource flags word used for every weight resource here.
constexpr int kBufFlags = 0x00020000;

}  // namespace mtp
