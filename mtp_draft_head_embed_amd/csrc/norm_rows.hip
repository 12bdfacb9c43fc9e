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
    __shared__ float red[32];
    const int b = blockIdx.x;
    const int H = a.H;
    const uint32_t tok = a.tokens[b];
    const bool tok_ok = tok < uint32_t(a.vocab);
    const uint16_t *erow = a.embed + (tok_ok ? size_t(tok) * size_t(H) : 0);
    uint16_t *dst = a.concat + size_t(b) * 2 * H;
    dual_norm(erow, tok_ok, a.enorm_w, a.hidden + size_t(b) * H, a.hnorm_w, H, a.eps, dst,
              dst + H, red);
}

// UB: partial sums loaded per batch (4 when S <= 4, as for the fused front's
// four K splits, so no split is read twice; else 8)
template <int UB>
__global__ __launch_bounds__(512) void sum_norm_kernel(SumNormArgs a)
{
    __shared__ float red[32];
    const int b = blockIdx.x;
    const int H = a.H;
    const int tid = threadIdx.x;
    if (a.zero_ctr && b == 0 && tid < kTilePools)
        a.zero_ctr[tid * (kCtrStride / 4)] = 0u;
    if (a.S == 0) {
        single_norm(a.x_in + size_t(b) * H, a.norm_w, H, a.eps, a.xn_out + size_t(b) * H, red);
        return;
    }
    // x = BF16(sum_s P[s][b]) in split order.  The partial sums are loaded
    // UB splits at a time for both pieces (a split past S re-reads the last
    // one and is not added), all issued before the first add, so a batch of
    // splits costs one memory latency rather than one per split.
    uint4 v[2], wv[2];
    float acc[2][8];
    bool in[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int j = (i * blockDim.x + tid) * 8;
        in[i] = j < H;
        wv[i] = make_uint4(0, 0, 0, 0);
        if (in[i] && a.xn_out)
            wv[i] = *reinterpret_cast<const uint4 *>(a.norm_w + j);
#pragma unroll
        for (int e = 0; e < 8; ++e)
            acc[i][e] = 0.f;
    }
    for (int sp0 = 0; sp0 < a.S; sp0 += UB) {
        float4 p[2][UB][2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            // a piece past H reads piece 0 of the row (never added)
            const int j = in[i] ? (i * blockDim.x + tid) * 8 : 0;
#pragma unroll
            for (int u = 0; u < UB; ++u) {
                const int sp = min(sp0 + u, a.S - 1);
                const float *src = a.P + (size_t(sp) * a.B + b) * H + j;
                p[i][u][0] = *reinterpret_cast<const float4 *>(src);
                p[i][u][1] = *reinterpret_cast<const float4 *>(src + 4);
            }
        }
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int u = 0; u < UB; ++u)
                if (sp0 + u < a.S) {
                    acc[i][0] += p[i][u][0].x; acc[i][1] += p[i][u][0].y;
                    acc[i][2] += p[i][u][0].z; acc[i][3] += p[i][u][0].w;
                    acc[i][4] += p[i][u][1].x; acc[i][5] += p[i][u][1].y;
                    acc[i][6] += p[i][u][1].z; acc[i][7] += p[i][u][1].w;
                }
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int j = (i * blockDim.x + tid) * 8;
        v[i] = make_uint4(0, 0, 0, 0);
        if (in[i]) {
            v[i] = make_uint4(pack_bf16x2(acc[i][0], acc[i][1]), pack_bf16x2(acc[i][2], acc[i][3]),
                              pack_bf16x2(acc[i][4], acc[i][5]), pack_bf16x2(acc[i][6], acc[i][7]));
            if (a.x_out)
                *reinterpret_cast<uint4 *>(a.x_out + size_t(b) * H + j) = v[i];
        }
    }
    if (!a.xn_out)
        return;
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const uint32_t w[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            ss = fmaf(bf16_lo(w[q]), bf16_lo(w[q]), ss);
            ss = fmaf(bf16_hi(w[q]), bf16_hi(w[q]), ss);
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
    const float rr = 1.0f / sqrtf(tot / float(H) + a.eps);  // as in the norms of common.hpp
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int j = (i * blockDim.x + tid) * 8;
        if (j < H) {
            const uint32_t xa[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
            const uint32_t wa[4] = {wv[i].x, wv[i].y, wv[i].z, wv[i].w};
            uint32_t o[4];
#pragma unroll
            for (int q = 0; q < 4; ++q)
                o[q] = pack_bf16x2((bf16_lo(xa[q]) * bf16_lo(wa[q])) * rr,
                                   (bf16_hi(xa[q]) * bf16_hi(wa[q])) * rr);
            *reinterpret_cast<uint4 *>(a.xn_out + size_t(b) * H + j) =
                make_uint4(o[0], o[1], o[2], o[3]);
        }
    }
}

hipError_t launch_front_concat(const FrontArgs &a, int batch, hipStream_t s)
{
    // 256 threads x 4 pieces of 8 cover H <= 8192 (measured 1% faster than
    // 512 threads for many rows)
    hipLaunchKernelGGL(front_concat_kernel, dim3(batch), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_sum_norm(const SumNormArgs &a, int batch, hipStream_t s)
{
    // 512 threads x 2 pieces of 8 cover H <= 8192
    if (a.S <= 4)
        hipLaunchKernelGGL(sum_norm_kernel<4>, dim3(batch), dim3(512), 0, s, a);
    else
        hipLaunchKernelGGL(sum_norm_kernel<8>, dim3(batch), dim3(512), 0, s, a);
    return hipGetLastError();
}

}  // namespace mtp
