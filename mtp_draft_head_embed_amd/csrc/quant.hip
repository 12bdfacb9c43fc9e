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
// The quotient.  With rs = fl32(1/s), t = fl32(w * rs) and the residual
// r = fma(-t, s, w), the corrected y = -fma(-r, rs, -t) has the same E4M3 code
// as clamp(fl32(w / s)) for every BF16 weight w with |w| <= amax and every row
// scale s >= 2^-100: checked exhaustively over all 1.04e9 such (amax, w) pairs
// (the negated form keeps the sign of a zero weight; below that scale the
// residual can underflow).  Rows with a smaller scale take the IEEE division.
//
// Codes: the hardware convert (v_cvt_pk_fp8_f32, two codes per instruction)
// rounds to the nearest E4M3FN value with ties to even on every float of
// magnitude <= 448, subnormal codes included, as the library's convert probe
// (mtp_probe_fp8_convert) checks over all 2.28e9 such floats.  So each element
// costs a multiply, two FMAs, a clamp and half a convert, with no per-element
// test or branch.
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace mtp {

typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2v __attribute__((ext_vector_type(2)));

__global__ void quant_flag_clear(uint32_t *flag) { *flag = 0u; }

// Lane l owns pieces of EPL consecutive elements: piece c holds elements
// c * 64 EPL + EPL l .. + EPL - 1 (EPL / 8 adjacent 16-byte loads), and its
// codes leave in one EPL-byte store.  As H is a multiple of 16, a piece lies
// wholly inside or wholly past the row; lanes past the end re-read the row's
// last EPL elements and store nothing.
template <int NP, int EPL>
struct RowRegs {
    uint4 w[NP][EPL / 8];
};

template <int NP, int EPL>
__device__ __forceinline__ void load_row(RowRegs<NP, EPL> &r, const uint16_t *__restrict__ L,
                                         int v, int H, int lane)
{
    const uint16_t *row = L + size_t(v) * size_t(H);
#pragma unroll
    for (int c = 0; c < NP; ++c) {
        const int j = min(c * 64 * EPL + lane * EPL, H - EPL);
#pragma unroll
        for (int h = 0; h < EPL / 8; ++h) {
            const u32x4v t =
                __builtin_nontemporal_load(reinterpret_cast<const u32x4v *>(row + j + 8 * h));
            r.w[c][h] = make_uint4(t.x, t.y, t.z, t.w);
        }
    }
}

template <int NP, int EPL>
__device__ __forceinline__ void quant_row(const RowRegs<NP, EPL> &r, int v, int H, int lane,
                                          uint8_t *__restrict__ q, float *__restrict__ scale,
                                          uint32_t *__restrict__ flag)
{
    uint32_t amax_bits = 0;  // |w| as bits: order-preserving for finite values
    bool bad = false;
#pragma unroll
    for (int c = 0; c < NP; ++c) {
        const bool in = c * 64 * EPL + lane * EPL < H;
#pragma unroll
        for (int h = 0; h < EPL / 8; ++h) {
            const uint32_t d[4] = {r.w[c][h].x, r.w[c][h].y, r.w[c][h].z, r.w[c][h].w};
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const uint32_t lo = in ? d[k] & 0x7FFFu : 0u;
                const uint32_t hi = in ? (d[k] >> 16) & 0x7FFFu : 0u;
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
    const float rs = 1.0f / s;
    // the corrected product gives the division's codes at these scales
    // (uniform per wave)
    const bool row_fast = s >= 0x1p-100f;
    if (lane == 0)
        scale[v] = s;
    auto encode = [&](auto fast) {
#pragma unroll
        for (int c = 0; c < NP; ++c) {
            const int j = c * 64 * EPL + lane * EPL;
            if (j < H) {
                float y[EPL];
#pragma unroll
                for (int k = 0; k < EPL; ++k) {
                    const uint4 &u = r.w[c][k >> 3];
                    const int wi = (k >> 1) & 3;
                    const uint32_t word = wi == 0 ? u.x : wi == 1 ? u.y : wi == 2 ? u.z : u.w;
                    const float x = (k & 1) ? bf16_hi(word) : bf16_lo(word);
                    float yk;
                    if constexpr (decltype(fast)::value) {
                        const float t = x * rs;
                        const float e = __builtin_fmaf(-t, s, x);
                        yk = -__builtin_fmaf(-e, rs, -t);
                    } else {
                        yk = x / s;
                    }
                    y[k] = fminf(fmaxf(yk, -448.0f), 448.0f);
                }
                uint32_t o[EPL / 4];
#pragma unroll
                for (int h = 0; h < EPL / 4; ++h) {
                    const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(y[4 * h], y[4 * h + 1], 0, false);
                    o[h] = uint32_t(
                        __builtin_amdgcn_cvt_pk_fp8_f32(y[4 * h + 2], y[4 * h + 3], lo, true));
                }
                uint8_t *dst = q + size_t(v) * size_t(H) + j;
                if constexpr (EPL == 16) {
                    const u32x4v ov = {o[0], o[1], o[2], o[3]};
                    __builtin_nontemporal_store(ov, reinterpret_cast<u32x4v *>(dst));
                } else {
                    const u32x2v ov = {o[0], o[1]};
                    __builtin_nontemporal_store(ov, reinterpret_cast<u32x2v *>(dst));
                }
            }
        }
    };
    if (row_fast)
        encode(std::true_type{});
    else
        encode(std::false_type{});
}

// RPW rows per wavefront, one wavefront per workgroup: every row's loads are
// issued before the first row is encoded, and the loads and code stores are
// non-temporal (each byte is touched once).
template <int NP, int EPL, int RPW>
__global__ __launch_bounds__(64) void quantize_kernel(const uint16_t *__restrict__ L, int V, int H,
                                                      uint8_t *__restrict__ q,
                                                      float *__restrict__ scale,
                                                      uint32_t *__restrict__ flag)
{
    const int lane = threadIdx.x;
    const int v0 = blockIdx.x * RPW;
    RowRegs<NP, EPL> r[RPW];
#pragma unroll
    for (int i = 0; i < RPW; ++i)
        load_row<NP, EPL>(r[i], L, min(v0 + i, V - 1), H, lane);
#pragma unroll
    for (int i = 0; i < RPW; ++i)
        if (v0 + i < V)
            quant_row<NP, EPL>(r[i], v0 + i, H, lane, q, scale, flag);
}

template <int EPL, int RPW>
static void launch_q(const uint16_t *L, int V, int H, uint8_t *q, float *scale, uint32_t *flag,
                     hipStream_t s)
{
    const int np = (H + 64 * EPL - 1) / (64 * EPL);
    const dim3 grid((V + RPW - 1) / RPW);
    constexpr int S = 8192 / (64 * EPL);  // pieces per lane at the largest H
    if (np <= S / 4)
        hipLaunchKernelGGL((quantize_kernel<S / 4, EPL, RPW>), grid, dim3(kWave), 0, s, L, V, H, q, scale, flag);
    else if (np <= S / 2)
        hipLaunchKernelGGL((quantize_kernel<S / 2, EPL, RPW>), grid, dim3(kWave), 0, s, L, V, H, q, scale, flag);
    else if (np <= 3 * S / 4)
        hipLaunchKernelGGL((quantize_kernel<3 * S / 4, EPL, RPW>), grid, dim3(kWave), 0, s, L, V, H, q, scale, flag);
    else
        hipLaunchKernelGGL((quantize_kernel<S, EPL, RPW>), grid, dim3(kWave), 0, s, L, V, H, q, scale, flag);
}

hipError_t launch_quantize(const uint16_t *L, int V, int H, uint8_t *q, float *scale,
                           uint32_t *flag, hipStream_t s)
{
    hipLaunchKernelGGL(quant_flag_clear, dim3(1), dim3(1), 0, s, flag);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    launch_q<8, 1>(L, V, H, q, scale, flag, s);
    return hipGetLastError();
}

}  // namespace mtp
