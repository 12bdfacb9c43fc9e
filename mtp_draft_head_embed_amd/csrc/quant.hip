// quant.hip -- the FP8 E4M3FN drafting copy of lm_head (metrale_model_arch/
// glm5next_mtp_head.rs, `head_fp8` field doc: an E4M3 copy of the head used
// only for drafting; quantisation may fail, and the caller keeps BF16).
//
// Per row v (one wavefront per row; the row stays in registers between the two
// passes):
//   a    = max_j |L[v][j]|                 exact on BF16 inputs
//   s_v  = a > 0 ? a / 448 : 1             IEEE f32 division (correctly rounded)
//   y    = clamp(L[v][j] / s_v, -448, 448) IEEE f32 division
//   q    = nearest E4M3FN code of y, ties to the even code, sign of zero kept
// A NaN or Inf weight raises a flag the host reads after the kernel.
//
// The encoder is integer arithmetic on the binary32 bits (no hardware convert),
// so its rounding is explicit:
//   |y| <  2^-6 : subnormal codes, M = rint(|y| * 2^9)  (0..8; 8 is 0x08, the
//                 smallest normal, which the code arithmetic gives by itself)
//   |y| >= 2^-6 : code = ((e + 7) << 3) + round-half-even of the 23-bit
//                 mantissa to 3 bits (a carry moves into the exponent field)
#include "common.hpp"
#include "kernels.hpp"

namespace mtp {

__device__ __forceinline__ uint32_t e4m3_encode(float y)
{
    const uint32_t u = __float_as_uint(y);
    const uint32_t sign = (u >> 24) & 0x80u;
    const uint32_t mag = u & 0x7FFFFFFFu;
    uint32_t code;
    if (mag < 0x3C800000u) {  // |y| < 2^-6
        // exact scaling by 2^9, then round to nearest even integer
        const float t = __uint_as_float(mag) * 512.0f;
        code = uint32_t(__builtin_rintf(t));
    } else {
        const uint32_t e = (mag >> 23) - 127u + 7u;  // biased E4M3 exponent, >= 1
        const uint32_t m = mag & 0x7FFFFFu;
        const uint32_t r = (m + 0x7FFFFu + ((m >> 20) & 1u)) >> 20;  // 0..8
        code = (e << 3) + r;
    }
    if (code > 0x7Eu)
        code = 0x7Eu;  // saturate (only reachable without the clamp)
    return sign | code;
}

__global__ void quant_flag_clear(uint32_t *flag) { *flag = 0u; }

__global__ __launch_bounds__(256) void quantize_kernel(const uint16_t *__restrict__ L, int V, int H,
                                                       uint8_t *__restrict__ q,
                                                       float *__restrict__ scale,
                                                       uint32_t *__restrict__ flag)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int v = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
    if (v >= V)
        return;  // whole wave exits together
    const uint16_t *row = L + size_t(v) * size_t(H);
    uint4 w[16];  // H <= 8192 = 16 chunks of 64 lanes x 8 elements
    uint32_t amax_bits = 0;  // |w| as bits: order-preserving for finite values
    bool bad = false;
#pragma unroll
    for (int c = 0; c < 16; ++c) {
        const int j = c * 512 + lane * 8;
        w[c] = make_uint4(0, 0, 0, 0);
        if (j < H) {
            w[c] = *reinterpret_cast<const uint4 *>(row + j);
            const uint32_t d[4] = {w[c].x, w[c].y, w[c].z, w[c].w};
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const uint32_t lo = d[k] & 0x7FFFu, hi = (d[k] >> 16) & 0x7FFFu;
                bad |= (lo >= 0x7F80u) | (hi >= 0x7F80u);
                amax_bits = max(amax_bits, max(lo, hi));
            }
        }
    }
    // wave max of the magnitude bits
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1)
        amax_bits = max(amax_bits, uint32_t(__shfl_xor(int(amax_bits), m, kWave)));
    if (bad)
        atomicOr(flag, 1u);
    const float amax = __uint_as_float(amax_bits << 16);
    const float s = amax > 0.f ? amax / 448.0f : 1.0f;
    if (lane == 0)
        scale[v] = s;
#pragma unroll
    for (int c = 0; c < 16; ++c) {
        const int j = c * 512 + lane * 8;
        if (j < H) {
            const uint32_t d[4] = {w[c].x, w[c].y, w[c].z, w[c].w};
            uint32_t o[2] = {0u, 0u};
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                float ylo = bf16_lo(d[k]) / s;
                float yhi = bf16_hi(d[k]) / s;
                ylo = fminf(fmaxf(ylo, -448.0f), 448.0f);
                yhi = fminf(fmaxf(yhi, -448.0f), 448.0f);
                const uint32_t pair = e4m3_encode(ylo) | (e4m3_encode(yhi) << 8);
                o[k >> 1] |= pair << ((k & 1) * 16);
            }
            *reinterpret_cast<uint2 *>(q + size_t(v) * size_t(H) + j) = make_uint2(o[0], o[1]);
        }
    }
}

hipError_t launch_quantize(const uint16_t *L, int V, int H, uint8_t *q, float *scale,
                           uint32_t *flag, hipStream_t s)
{
    hipLaunchKernelGGL(quant_flag_clear, dim3(1), dim3(1), 0, s, flag);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    const int rows_per_block = 4;
    hipLaunchKernelGGL(quantize_kernel, dim3((V + rows_per_block - 1) / rows_per_block), dim3(256),
                       0, s, L, V, H, q, scale, flag);
    return hipGetLastError();
}

}  // namespace mtp
