// norm_rows.hip -- per-sequence vector work of the batched (B >= 2) sweep,
// one workgroup per sequence:
//   * front_concat_kernel: concat[b] = [enorm(embed[tokens[b]]) | hnorm(hidden[b])]
//     (metrale_model_arch/glm5next_mtp_head.rs, `forward_one`: the embedding
//     row read by pointer, then the two vanilla norms into the [2, H] scratch).
//   * sum_norm_kernel: x[b] = BF16(sum over the eh_proj K-splits, in split
//     order) and xn[b] = BF16(shared_head.norm(x[b])) (same page: the final
//     norm ahead of the head).
// The single-sequence sweep fuses these into the GEMV prologues instead.
#include "common.hpp"
#include "kernels.hpp"

namespace mtp {

__global__ __launch_bounds__(256) void front_concat_kernel(FrontArgs a)
{
    __shared__ float red[16];
    const int b = blockIdx.x;
    const int H = a.H;
    const uint32_t tok = a.tokens[b];
    const bool tok_ok = tok < uint32_t(a.vocab);
    const uint16_t *erow = a.embed + (tok_ok ? size_t(tok) * size_t(H) : 0);
    uint16_t *dst = a.concat + size_t(b) * 2 * H;
    uint4 v[4];
    float ss = block_sumsq(erow, H, tok_ok, v, red);
    norm_to_lds(v, a.enorm_w, H, sqrtf(ss / float(H) + a.eps), dst);
    ss = block_sumsq(a.hidden + size_t(b) * H, H, true, v, red);
    norm_to_lds(v, a.hnorm_w, H, sqrtf(ss / float(H) + a.eps), dst + H);
}

__global__ __launch_bounds__(256) void sum_norm_kernel(SumNormArgs a)
{
    __shared__ float red[16];
    const int b = blockIdx.x;
    const int H = a.H;
    const int tid = threadIdx.x;
    uint4 v[4];
    if (a.S > 0) {
        // x = BF16(sum_s P[s][b]) in split order
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int j = (i * blockDim.x + tid) * 8;
            v[i] = make_uint4(0, 0, 0, 0);
            if (j < H) {
                float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
                for (int sp = 0; sp < a.S; ++sp) {
                    const float *src = a.P + (size_t(sp) * a.B + b) * H + j;
                    const float4 p0 = *reinterpret_cast<const float4 *>(src);
                    const float4 p1 = *reinterpret_cast<const float4 *>(src + 4);
                    acc[0] += p0.x; acc[1] += p0.y; acc[2] += p0.z; acc[3] += p0.w;
                    acc[4] += p1.x; acc[5] += p1.y; acc[6] += p1.z; acc[7] += p1.w;
                }
                v[i] = make_uint4(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]),
                                  pack_bf16x2(acc[4], acc[5]), pack_bf16x2(acc[6], acc[7]));
                if (a.x_out)
                    *reinterpret_cast<uint4 *>(a.x_out + size_t(b) * H + j) = v[i];
            }
        }
        if (!a.xn_out)
            return;
        // sum of squares of the rounded x, same order as block_sumsq
        float ss = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t w[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float lo = bf16_lo(w[q]), hi = bf16_hi(w[q]);
                ss = fmaf(lo, lo, ss);
                ss = fmaf(hi, hi, ss);
            }
        }
        ss = wave_sum(ss);
        __syncthreads();
        if ((tid & (kWave - 1)) == 0)
            red[tid / kWave] = ss;
        __syncthreads();
        float tot = 0.f;
        for (int w = 0; w < int(blockDim.x / kWave); ++w)
            tot += red[w];
        norm_to_lds(v, a.norm_w, H, sqrtf(tot / float(H) + a.eps), a.xn_out + size_t(b) * H);
    } else {
        const float ss = block_sumsq(a.x_in + size_t(b) * H, H, true, v, red);
        norm_to_lds(v, a.norm_w, H, sqrtf(ss / float(H) + a.eps), a.xn_out + size_t(b) * H);
    }
}

hipError_t launch_front_concat(const FrontArgs &a, int batch, hipStream_t s)
{
    hipLaunchKernelGGL(front_concat_kernel, dim3(batch), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_sum_norm(const SumNormArgs &a, int batch, hipStream_t s)
{
    hipLaunchKernelGGL(sum_norm_kernel, dim3(batch), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace mtp
