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
// The quotient: t = w * (1/s), with 1/s correctly rounded once per row, is
// within 2^-23 of w/s relative, so within 3 units in the last place of t from
// fl32(w/s).  Rounding to E4M3 only changes where a rounding boundary (a
// midpoint between two codes) lies between them, so t gives the same code as
// fl32(w/s) unless t lies within a few units of a midpoint (bits 0..19 of the
// mantissa near 0x80000) or in the E4M3 subnormal range; those elements, and
// whole rows whose 1/s would not be a normal float, take the IEEE division.
// That keeps the codes those of the correctly rounded quotient while most
// elements cost a multiply instead of a division sequence.
//
// Codes: an element decided by t is no tie and no near tie, so the hardware
// FP8 convert (round to nearest) gives its code.  The elements that take the
// division go through an integer encoder on the binary32 bits, so the ties
// and the subnormal range have explicit rounding:
//   |y| <  2^-6 : subnormal codes, M = rint(|y| * 2^9)  (0..8; 8 is 0x08, the
//                 smallest normal, which the code arithmetic gives by itself)
//   |y| >= 2^-6 : code = ((e + 7) << 3) + round-half-even of the 23-bit
//                 mantissa to 3 bits (a carry moves into the exponent field)
#include "common.hpp"
#include "kernels.hpp"

namespace mtp {

typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2v __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t e4m3_encode(float y)
{
    const uint32_t u = __float_as_uint(y);
    const uint32_t sign = (u >> 24) & 0x80u;
    const uint32_t mag = u & 0x7FFFFFFFu;
    // |y| < 2^-6: exact scaling by 2^9, then round to the nearest even integer
    const uint32_t sub = uint32_t(__builtin_rintf(__uint_as_float(mag) * 512.0f));
    // |y| >= 2^-6: biased E4M3 exponent (>= 1) and the 23-bit mantissa rounded
    // half to even to 3 bits (0..8; 8 carries into the exponent)
    const uint32_t e = (mag >> 23) - 127u + 7u;
    const uint32_t m = mag & 0x7FFFFFu;
    const uint32_t r = (m + 0x7FFFFu + ((m >> 20) & 1u)) >> 20;
    uint32_t code = mag < 0x3C800000u ? sub : (e << 3) + r;
    if (code > 0x7Eu)
        code = 0x7Eu;  // saturate (only reachable without the clamp)
    return sign | code;
}

__global__ void quant_flag_clear(uint32_t *flag) { *flag = 0u; }

// Loads one row's NC chunks (lane l holds elements c * 512 + 8l .. + 7 of
// chunk c).  Lanes past the end of a ragged last chunk re-read the row's last
// 16 bytes (H % 16 == 0, so that address is aligned); quant_row drops them.
template <int NC>
__device__ __forceinline__ void load_row(uint4 (&w)[NC], const uint16_t *__restrict__ L, int v,
                                         int H, int lane)
{
    const uint16_t *row = L + size_t(v) * size_t(H);
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        const u32x4v t = __builtin_nontemporal_load(
            reinterpret_cast<const u32x4v *>(row + min(c * 512 + lane * 8, H - 8)));
        w[c] = make_uint4(t.x, t.y, t.z, t.w);
    }
}

template <int NC>
__device__ __forceinline__ void quant_row(const uint4 (&w)[NC], int v, int H, int lane,
                                          uint8_t *__restrict__ q, float *__restrict__ scale,
                                          uint32_t *__restrict__ flag)
{
    uint32_t amax_bits = 0;  // |w| as bits: order-preserving for finite values
    bool bad = false;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        const bool in = c * 512 + lane * 8 < H;
        const uint32_t d[4] = {w[c].x, w[c].y, w[c].z, w[c].w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint32_t lo = in ? d[k] & 0x7FFFu : 0u;
            const uint32_t hi = in ? (d[k] >> 16) & 0x7FFFu : 0u;
            bad |= (lo >= 0x7F80u) | (hi >= 0x7F80u);
            amax_bits = max(amax_bits, max(lo, hi));
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
    const float rs = 1.0f / s;
    // 1/s normal and finite: the relative bound on t holds (uniform per wave)
    const bool row_fast = s >= 0x1p-120f && s <= 0x1p120f;
    if (lane == 0)
        scale[v] = s;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        const int j = c * 512 + lane * 8;
        if (j < H) {
            const uint32_t d[4] = {w[c].x, w[c].y, w[c].z, w[c].w};
            float t[8];
            bool unsure = !row_fast;
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const float x = (k & 1) ? bf16_hi(d[k >> 1]) : bf16_lo(d[k >> 1]);
                t[k] = fminf(fmaxf(x * rs, -448.0f), 448.0f);
                const uint32_t mag = __float_as_uint(t[k]) & 0x7FFFFFFFu;
                // below 2^-6, or within 16 units of a midpoint: not decided by t
                unsure |= (mag < 0x3C800000u) | (((mag & 0xFFFFFu) - 0x7FFF0u) <= 32u);
            }
            // a sure t lies in E4M3's normal range, at least 16 units from every
            // midpoint, so any round-to-nearest conversion gives its code; the
            // hardware one packs two codes per instruction, in element order
            uint32_t o[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(t[4 * h], t[4 * h + 1], 0, false);
                o[h] = uint32_t(__builtin_amdgcn_cvt_pk_fp8_f32(t[4 * h + 2], t[4 * h + 3], lo, true));
            }
            if (unsure) {
                o[0] = o[1] = 0u;
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    const float x = (k & 1) ? bf16_hi(d[k >> 1]) : bf16_lo(d[k >> 1]);
                    o[k >> 2] |= e4m3_encode(fminf(fmaxf(x / s, -448.0f), 448.0f)) << ((k & 3) * 8);
                }
            }
            const u32x2v ov = {o[0], o[1]};
            __builtin_nontemporal_store(ov, reinterpret_cast<u32x2v *>(q + size_t(v) * size_t(H) + j));
        }
    }
}

// One wavefront per workgroup and per row: a finished wave frees its slot at
// once, and the row's loads and code stores are non-temporal (each byte is
// touched once).  Measured against a persistent grid whose waves prefetch
// their next row while encoding the current one: that grid was slower.
template <int NC>
__global__ __launch_bounds__(64) void quantize_kernel(const uint16_t *__restrict__ L, int V, int H,
                                                      uint8_t *__restrict__ q,
                                                      float *__restrict__ scale,
                                                      uint32_t *__restrict__ flag)
{
    const int lane = threadIdx.x;
    const int v = blockIdx.x;
    uint4 w[NC];
    load_row<NC>(w, L, v, H, lane);
    quant_row<NC>(w, v, H, lane, q, scale, flag);
}

hipError_t launch_quantize(const uint16_t *L, int V, int H, uint8_t *q, float *scale,
                           uint32_t *flag, hipStream_t s)
{
    hipLaunchKernelGGL(quant_flag_clear, dim3(1), dim3(1), 0, s, flag);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    const int nch = (H + 511) / 512;
    if (nch <= 4)
        hipLaunchKernelGGL(quantize_kernel<4>, dim3(V), dim3(kWave), 0, s, L, V, H, q, scale, flag);
    else if (nch <= 8)
        hipLaunchKernelGGL(quantize_kernel<8>, dim3(V), dim3(kWave), 0, s, L, V, H, q, scale, flag);
    else if (nch <= 12)
        hipLaunchKernelGGL(quantize_kernel<12>, dim3(V), dim3(kWave), 0, s, L, V, H, q, scale, flag);
    else
        hipLaunchKernelGGL(quantize_kernel<16>, dim3(V), dim3(kWave), 0, s, L, V, H, q, scale, flag);
    return hipGetLastError();
}

}  // namespace mtp
