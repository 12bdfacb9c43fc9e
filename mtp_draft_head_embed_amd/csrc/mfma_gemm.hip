// mfma_gemm.hip -- the batched (B >= 2) sweep: Y[b][n] = sum_k A[b][k] * W[n][k]
// on gfx950 matrix cores, for B independent sequences sharing the weights.
//
// Used for lm_head (`dense_gemv` / `dense_gemv_fp8w` of
// metrale_model_arch/glm5next_mtp_head.rs, `forward_one`, run for B sequences
// at once) with the argmax-partials epilogue, and for eh_proj with split-K and
// an FP32 partial-sum epilogue.  Every weight byte is read once per call for
// all B sequences; at B = 16 this is 16 multiply-adds per weight, more than
// the vector ALUs can sustain at HBM rate, hence MFMA.  It is still
// bandwidth-bound (32 flop per FP8 byte is far below the MFMA ridge).
//
// Shape of the work:
//   * v_mfma_f32_16x16x32_bf16, D[m][n] += A[m][k] B[k][n], with m = sequence
//     (16 per batch tile, padded with zero rows) and n = weight row (16 per
//     tile).  Lane l supplies A row l%16 and W row l%16 for its k-slot group
//     l/16; D lane l holds m = 4*(l/16) + i, n = l%16.  Both operands take
//     the same columns for a given (lane group, element), so the order in
//     which k is split over lanes does not change the sum's terms.
//   * The activations of a K-chunk are staged in LDS ([16*NBT][KC + 8] BF16,
//     rows padded by 16 B so the 16 lanes of a row group hit distinct banks);
//     each wave owns up to MAXT 16-row weight tiles per pass and keeps their
//     accumulators in registers across the chunks.
//   * FP8 codes are decoded to BF16 in registers (v_cvt_scalef32_pk_bf16_fp8
//     with scale 1, exact for every E4M3FN value); the per-row scale multiplies
//     the FP32 sum once, as the FP8 head defines it.
//   * Weights stream with 16-byte non-temporal loads, UK k-steps in flight.
#include "common.hpp"
#include "kernels.hpp"

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

__device__ __forceinline__ bf16x8 as_bf16x8(const uint4 &u)
{
    bf16x8 r;
    __builtin_memcpy(&r, &u, 16);
    return r;
}

// 8 E4M3FN codes (two dwords) -> 8 BF16 values, in order.
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

template <bool FP8, int EPI, int NBT, int MAXT, int UK>
__global__ __launch_bounds__(256) void mfma_gemm_kernel(MfmaArgs a)
{
    extern __shared__ uint4 lds_raw[];
    uint16_t *As = reinterpret_cast<uint16_t *>(lds_raw);
    constexpr int BP = 16 * NBT;  // padded batch rows
    const int lane = threadIdx.x & (kWave - 1);
    const int wid = threadIdx.x / kWave;
    const int nl = lane & 15;  // row within a tile (weights) / batch row (activations)
    const int g = lane >> 4;   // k-slot group
    const int KC = a.KC;
    const int rs = KC + 8;     // LDS row stride in BF16 elements
    const int B = a.B;
    const int N = a.N;
    const int K = a.K;
    const int split = blockIdx.y;
    const int k_begin = split * a.Ks;
    const int k_end = min(K, k_begin + a.Ks);
    const int T = (N + 15) / 16;
    const int Wt = gridDim.x * 4;
    const int gw = blockIdx.x * 4 + wid;
    const char *Wb = reinterpret_cast<const char *>(a.W);
    const size_t wrow = FP8 ? size_t(K) : size_t(K) * 2;  // bytes per weight row

    // padded activation rows stay zero for the whole kernel
    for (int i = threadIdx.x; i < (BP - B) * (rs / 8); i += blockDim.x)
        *reinterpret_cast<uint4 *>(As + size_t(B) * rs + size_t(i) * 8) = make_uint4(0, 0, 0, 0);

    float best_v[NBT][4];
    uint32_t best_i[NBT][4];
#pragma unroll
    for (int bt = 0; bt < NBT; ++bt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            best_v[bt][i] = -INFINITY;
            best_i[bt][i] = 0xFFFFFFFFu;
        }

    // tile groups: every wave of the workgroup runs the same number of passes
    // (the workgroup's first wave has the most tiles) so the barriers match
    const int first_w = blockIdx.x * 4;
    const int tiles_w0 = first_w < T ? (T - first_w + Wt - 1) / Wt : 0;
    const int npass = (tiles_w0 + MAXT - 1) / MAXT;

    for (int pass = 0; pass < npass; ++pass) {
        f32x4 acc[MAXT][NBT];
#pragma unroll
        for (int j = 0; j < MAXT; ++j)
#pragma unroll
            for (int bt = 0; bt < NBT; ++bt)
                acc[j][bt] = f32x4{0.f, 0.f, 0.f, 0.f};

        for (int kc0 = k_begin; kc0 < k_end; kc0 += KC) {
            const int kc_len = min(KC, k_end - kc0);  // a multiple of 16
            __syncthreads();  // previous chunk's LDS reads are done
            for (int i = threadIdx.x; i < B * (KC / 8); i += blockDim.x) {
                const int bb = i / (KC / 8);
                const int c = (i - bb * (KC / 8)) * 8;
                uint4 v = make_uint4(0, 0, 0, 0);
                if (c < kc_len)
                    v = *reinterpret_cast<const uint4 *>(a.A + size_t(bb) * K + kc0 + c);
                *reinterpret_cast<uint4 *>(As + size_t(bb) * rs + c) = v;
            }
            __syncthreads();

            // k-steps of 32 columns.  FP8 loads cover a pair of steps (64
            // columns), so the FP8 count is a whole number of pairs; columns
            // past the chunk are zero in LDS and not loaded from HBM.
            const int nsteps = FP8 ? 2 * ((kc_len + 63) / 64) : (kc_len + 31) / 32;
#pragma unroll
            for (int j = 0; j < MAXT; ++j) {
                const int t = gw + (pass * MAXT + j) * Wt;
                if (t >= T)
                    continue;  // uniform across the wave
                const int row = t * 16 + nl;
                const bool row_ok = row < N;
                const char *wr = Wb + size_t(row_ok ? row : 0) * wrow;
#pragma unroll 1
                for (int s0 = 0; s0 < nsteps; s0 += UK) {
                    bf16x8 wf[UK];
                    if (!FP8) {
                        uint4 raw[UK];
#pragma unroll
                        for (int u = 0; u < UK; ++u) {
                            const int col = kc0 + (s0 + u) * 32 + g * 8;
                            raw[u] = make_uint4(0, 0, 0, 0);
                            if (row_ok && s0 + u < nsteps && col < k_end)
                                raw[u] = ld_nt16(wr + size_t(col) * 2);
                        }
#pragma unroll
                        for (int u = 0; u < UK; ++u)
                            wf[u] = as_bf16x8(raw[u]);
                    } else {
                        // step pair p = (s0 + u) / 2: lane group g reads codes
                        // [64p + 16g, +16); the even step takes the first 8
                        uint4 raw[UK / 2];
#pragma unroll
                        for (int u = 0; u < UK / 2; ++u) {
                            const int col = kc0 + ((s0 >> 1) + u) * 64 + g * 16;
                            raw[u] = make_uint4(0, 0, 0, 0);
                            if (row_ok && s0 + 2 * u < nsteps && col < k_end)
                                raw[u] = ld_nt16(wr + size_t(col));
                        }
#pragma unroll
                        for (int u = 0; u < UK / 2; ++u) {
                            wf[2 * u] = fp8x8_to_bf16(raw[u].x, raw[u].y);
                            wf[2 * u + 1] = fp8x8_to_bf16(raw[u].z, raw[u].w);
                        }
                    }
#pragma unroll
                    for (int u = 0; u < UK; ++u) {
                        if (s0 + u < nsteps) {
                            // LDS column of this lane's 8 activations for step s0+u
                            const int lc = FP8 ? ((s0 + u) >> 1) * 64 + g * 16 + ((s0 + u) & 1) * 8
                                               : (s0 + u) * 32 + g * 8;
#pragma unroll
                            for (int bt = 0; bt < NBT; ++bt) {
                                const uint4 av = *reinterpret_cast<const uint4 *>(
                                    As + size_t(bt * 16 + nl) * rs + lc);
                                acc[j][bt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                    as_bf16x8(av), wf[u], acc[j][bt], 0, 0, 0);
                            }
                        }
                    }
                }
            }
        }

        // ---- epilogue for this pass's tiles ----------------------------------
#pragma unroll
        for (int j = 0; j < MAXT; ++j) {
            const int t = gw + (pass * MAXT + j) * Wt;
            if (t >= T)
                continue;
            const int row = t * 16 + nl;
            if (row >= N)
                continue;
            const float sc = (FP8 && EPI == EPI_ARGMAX) ? a.scale[row] : 1.0f;
#pragma unroll
            for (int bt = 0; bt < NBT; ++bt) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int bb = bt * 16 + g * 4 + i;
                    if (bb >= B)
                        continue;
                    const float z = acc[j][bt][i];
                    if (EPI == EPI_STORE) {
                        a.out_f32[(size_t(split) * B + bb) * N + row] = z;
                    } else {
                        const uint32_t lb = f32_to_bf16_bits(FP8 ? z * sc : z);
                        if (a.logits)
                            a.logits[size_t(bb) * N + row] = uint16_t(lb);
                        const float lv = __uint_as_float(lb << 16);
                        if (better(lv, uint32_t(row), best_v[bt][i], best_i[bt][i])) {
                            best_v[bt][i] = lv;
                            best_i[bt][i] = uint32_t(row);
                        }
                    }
                }
            }
        }
    }

    if (EPI == EPI_ARGMAX) {
        // reduce over the 16 lanes that share a batch row group (lane bits 0-3)
#pragma unroll
        for (int bt = 0; bt < NBT; ++bt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int m = 1; m < 16; m <<= 1) {
                    const float ov = __shfl_xor(best_v[bt][i], m, kWave);
                    const uint32_t oi = __shfl_xor(best_i[bt][i], m, kWave);
                    if (better(ov, oi, best_v[bt][i], best_i[bt][i])) {
                        best_v[bt][i] = ov;
                        best_i[bt][i] = oi;
                    }
                }
        __syncthreads();  // LDS is reused for the cross-wave reduction
        float *rv = reinterpret_cast<float *>(lds_raw);
        uint32_t *ri = reinterpret_cast<uint32_t *>(rv + 4 * BP);
        if (nl == 0) {
#pragma unroll
            for (int bt = 0; bt < NBT; ++bt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    rv[wid * BP + bt * 16 + g * 4 + i] = best_v[bt][i];
                    ri[wid * BP + bt * 16 + g * 4 + i] = best_i[bt][i];
                }
        }
        __syncthreads();
        for (int bb = threadIdx.x; bb < B; bb += blockDim.x) {
            float bv = rv[bb];
            uint32_t bi = ri[bb];
            for (int w = 1; w < 4; ++w)
                if (better(rv[w * BP + bb], ri[w * BP + bb], bv, bi)) {
                    bv = rv[w * BP + bb];
                    bi = ri[w * BP + bb];
                }
            a.partials[size_t(bb) * kMaxHeadBlocks + blockIdx.x] = Partial{bv, bi};
        }
    }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------

static int g_lds_limit = 0;  // per-block LDS bytes the device allows (queried once)

static int lds_limit()
{
    if (g_lds_limit == 0) {
        int dev = 0, v = 0;
        if (hipGetDevice(&dev) == hipSuccess &&
            hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) == hipSuccess &&
            v > 0)
            g_lds_limit = v;
        else
            g_lds_limit = 65536;
    }
    return g_lds_limit;
}

// Chunk width: the largest multiple of 64 whose [16*NBT][KC+8] BF16 tile fits
// the LDS budget, then evened out over the chunks a split needs.
static int chunk_cols(int nbt, int klen)
{
    const int budget = min(lds_limit(), 65536) - 1024;
    int kc_max = (budget / (16 * nbt * 2) - 8) / 64 * 64;
    if (kc_max < 64)
        kc_max = 64;
    const int nch = (klen + kc_max - 1) / kc_max;
    int kc = ((klen + nch - 1) / nch + 63) / 64 * 64;
    return kc < 64 ? 64 : kc;
}

template <bool FP8, int EPI, int NBT>
static hipError_t launch_mfma_nbt(MfmaArgs a, int grid, int splits, hipStream_t s)
{
    constexpr int MAXT = NBT == 1 ? 8 : (NBT == 2 ? 4 : 2);
    constexpr int UK = FP8 ? 16 : 8;
    a.KC = chunk_cols(NBT, a.Ks);
    size_t lds = size_t(16 * NBT) * size_t(a.KC + 8) * 2;
    const size_t red = size_t(4 * 16 * NBT) * 8;
    if (lds < red)
        lds = red;
    hipLaunchKernelGGL((mfma_gemm_kernel<FP8, EPI, NBT, MAXT, UK>), dim3(grid, splits), dim3(256),
                       lds, s, a);
    return hipGetLastError();
}

template <bool FP8, int EPI>
static hipError_t launch_mfma(const MfmaArgs &a, int grid, int splits, hipStream_t s)
{
    const int nbt = (a.B + 15) / 16;
    switch (nbt) {
    case 1: return launch_mfma_nbt<FP8, EPI, 1>(a, grid, splits, s);
    case 2: return launch_mfma_nbt<FP8, EPI, 2>(a, grid, splits, s);
    case 3: return launch_mfma_nbt<FP8, EPI, 3>(a, grid, splits, s);
    default: return launch_mfma_nbt<FP8, EPI, 4>(a, grid, splits, s);
    }
}

EhSplit eh_split(int hidden)
{
    // aim for about 2048 waves: one 16-row tile per wave, K split S ways
    const int T = (hidden + 15) / 16;
    const int K = 2 * hidden;
    int S = (2048 + T - 1) / T;
    if (S < 1)
        S = 1;
    if (S > 32)
        S = 32;
    int Ks = ((K + S - 1) / S + 63) / 64 * 64;
    S = (K + Ks - 1) / Ks;
    return EhSplit{S, Ks};
}

int eh_split_count(int hidden) { return eh_split(hidden).S; }

hipError_t launch_eh_proj_mfma(const MfmaArgs &a_in, hipStream_t s)
{
    MfmaArgs a = a_in;
    const EhSplit sp = eh_split(a.N);
    a.Ks = sp.Ks;
    const int T = (a.N + 15) / 16;
    int grid = (T + 3) / 4;  // one tile per wave
    if (grid > kMaxHeadBlocks)
        grid = kMaxHeadBlocks;
    return launch_mfma<false, EPI_STORE>(a, grid, sp.S, s);
}

hipError_t launch_head_mfma(const MfmaArgs &a_in, bool fp8, int *grid_out, hipStream_t s)
{
    MfmaArgs a = a_in;
    a.Ks = a.K;
    const int T = (a.N + 15) / 16;
    int grid = device_cu_count() * 2;
    const int need = (T + 3) / 4;
    if (grid > need)
        grid = need;
    if (grid > kMaxHeadBlocks)
        grid = kMaxHeadBlocks;
    if (grid < 1)
        grid = 1;
    *grid_out = grid;
    return fp8 ? launch_mfma<true, EPI_ARGMAX>(a, grid, 1, s)
               : launch_mfma<false, EPI_ARGMAX>(a, grid, 1, s);
}

}  // namespace mtp
