// ctx_gemm.hip -- the drafter's context rows (metrale_model_arch/
// glm5next_mtp_head.rs, `rows_impl`): T prompt or catch-up rows through the
// front half, row r pairing embed(tokens[r + 1]) with hiddens[r]:
//
//   x[r] = BF16(eh_proj . [enorm(embed[tokens[r+1]]) | hnorm(hiddens[r])])
//
// The page stops each row at the block's KV-cache write (out of scope here).
// With T rows, eh_proj is a dense GEMM C[T][H] = A[T][2H] . W[H][2H]^T with
// both operands K-contiguous; beyond a few hundred rows it is bound by the
// matrix cores, so it is tiled for MFMA:
//   * 128 x 128 output tile per 256-thread workgroup, four waves of 64 x 64,
//     each a 4 x 4 grid of v_mfma_f32_16x16x32_bf16 accumulators;
//   * K in steps of 64 through LDS, double-buffered: the next step's global
//     loads (8 lanes x 16 B per row, whole 128-B lines) are in registers while
//     the current step is multiplied, then written to the other buffer;
//   * LDS rows padded to 72 BF16 (144 B) so the 16 lanes of a fragment read
//     hit disjoint banks;
//   * partial tiles (T or H not a multiple of 128, 2H not of 64) load zeros;
//   * with few tiles (a skinny T) K is split over blockIdx.z so that about
//     512 workgroups fill the 256 CUs; each split writes an FP32 partial tile
//     and the splits are summed in split order by the batched path's
//     sum-and-round kernel.
// Sums are FP32 in a fixed k order, so results do not depend on timing.
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"
#include "ctx_gemm.hpp"

namespace mtp {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int BK = 64;
constexpr int LDR = BK + 8;  // LDS row stride, BF16 elements

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// 16-byte raw buffer load; an offset at or past the resource's size returns 0
__device__ __forceinline__ uint4 ld_b128(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, int(off), 0, 0);
    return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ bf16x8_t to_bf16x8(const uint4 &u)
{
    bf16x8_t r;
    __builtin_memcpy(&r, &u, 16);
    return r;
}

}  // namespace

// BM x BN output tile per workgroup of WM x WN waves; each wave owns a
// (BM/WM) x (BN/WN) block of 16 x 16 MFMA accumulators.
template <int BM, int BN, int WM, int WN>
__global__ __launch_bounds__(WM *WN * 64) void ctx_gemm_kernel(const uint16_t *__restrict__ A,
                                                               const uint16_t *__restrict__ W,
                                                               uint16_t *__restrict__ C,
                                                               float *__restrict__ P, int M, int N,
                                                               int K, int Ks)
{
    constexpr int NT = WM * WN * 64;
    constexpr int FM = BM / WM / 16, FN = BN / WN / 16;
    constexpr int RPP = NT / 8;  // tile rows one pass of global loads covers
    constexpr int PA = BM / RPP, PW = BN / RPP;
    static_assert(BM % RPP == 0 && BN % RPP == 0, "tile rows must be whole passes");
    extern __shared__ uint4 ctx_lds[];
    uint16_t *sA0 = reinterpret_cast<uint16_t *>(ctx_lds);
    uint16_t *sW0 = sA0 + 2 * BM * LDR;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wid = tid >> 6;
    const int wm = wid / WN, wn = wid % WN;
    const int nl = lane & 15, g = lane >> 4;
    const int m0 = blockIdx.y * BM;
    const int n0 = blockIdx.x * BN;
    const int k_begin = blockIdx.z * Ks;
    const int k_end = min(K, k_begin + Ks);

    // global -> register staging: thread t covers rows t/8 + RPP p, columns
    // (t%8)*8 .. +8 of the 64-column step.  The tile's rows form a buffer
    // resource, so rows past M read as zero without a branch, and a column
    // past the split takes an offset beyond the resource (zero as well).
    const int lr = tid >> 3;
    const int lc = (tid & 7) * 8;
    const uint32_t rowb = uint32_t(K) * 2;  // bytes per row
    const __amdgpu_buffer_rsrc_t arsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(A) + size_t(m0) * K, 0, int(uint32_t(min(BM, M - m0)) * rowb),
        0x00020000);
    const __amdgpu_buffer_rsrc_t wrsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(W) + size_t(n0) * K, 0, int(uint32_t(min(BN, N - n0)) * rowb),
        0x00020000);
    const uint32_t toff = uint32_t(lr) * rowb + uint32_t(lc) * 2;
    // two register sets: the loads of step k + 2 are issued before step k is
    // multiplied, so each load has about two steps of MFMA work to land
    uint4 ra[2][PA], rw[2][PW];
    auto gload = [&](int set, int k0) {
        const uint32_t o = (k0 + lc < k_end) ? toff + uint32_t(k0) * 2 : 0x80000000u;
#pragma unroll
        for (int p = 0; p < PA; ++p)
            ra[set][p] = ld_b128(arsrc, o + uint32_t(RPP * p) * rowb);
#pragma unroll
        for (int p = 0; p < PW; ++p)
            rw[set][p] = ld_b128(wrsrc, o + uint32_t(RPP * p) * rowb);
    };
    auto sstore = [&](int set, int buf) {
        uint16_t *sA = sA0 + buf * BM * LDR;
        uint16_t *sW = sW0 + buf * BN * LDR;
#pragma unroll
        for (int p = 0; p < PA; ++p)
            *reinterpret_cast<uint4 *>(&sA[(lr + RPP * p) * LDR + lc]) = ra[set][p];
#pragma unroll
        for (int p = 0; p < PW; ++p)
            *reinterpret_cast<uint4 *>(&sW[(lr + RPP * p) * LDR + lc]) = rw[set][p];
    };

    f32x4_t acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
            acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    auto mma_step = [&](int buf) {
        const uint16_t *sA = sA0 + buf * BM * LDR;
        const uint16_t *sW = sW0 + buf * BN * LDR;
#pragma unroll
        for (int sub = 0; sub < BK / 32; ++sub) {
            const int kc = sub * 32 + g * 8;
            bf16x8_t af[FM], wf[FN];
#pragma unroll
            for (int i = 0; i < FM; ++i)
                af[i] = to_bf16x8(*reinterpret_cast<const uint4 *>(
                    &sA[((wm * FM + i) * 16 + nl) * LDR + kc]));
#pragma unroll
            for (int j = 0; j < FN; ++j)
                wf[j] = to_bf16x8(*reinterpret_cast<const uint4 *>(
                    &sW[((wn * FN + j) * 16 + nl) * LDR + kc]));
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], wf[j], acc[i][j],
                                                                        0, 0, 0);
        }
    };

    // step k lives in register set k & 1 and LDS buffer k & 1
    const int nk = (k_end - k_begin + BK - 1) / BK;
    gload(0, k_begin);
    gload(1, k_begin + BK);
    sstore(0, 0);
    __syncthreads();
    // Register sets and LDS buffers alternate, so the loop runs in pairs to
    // keep every register index a compile-time constant.  Loads and stores
    // are unconditional (past the split they read zeros and fill a buffer that
    // is never read), so every path holds the same loads in flight and each
    // store waits only for its own set.
    auto step = [&](int kt, auto bc) {
        constexpr int b = decltype(bc)::value;
        gload(b, k_begin + (kt + 2) * BK);  // set b was stored to LDS last step
        __builtin_amdgcn_sched_barrier(0);  // issue the loads before the MFMAs
        mma_step(b);
        sstore(b ^ 1, b ^ 1);
        __syncthreads();
    };
    // an odd count gets one step past the split: zeros, which leave the sums
    // unchanged (the accumulators start at +0)
    for (int kt = 0; kt < nk; kt += 2) {
        step(kt, std::integral_constant<int, 0>{});
        step(kt + 1, std::integral_constant<int, 1>{});
    }

    // lane (g, n) holds rows 4g..4g+3 of column n of each 16 x 16 tile
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int col = n0 + (wn * FN + j) * 16 + nl;
            if (col >= N)
                continue;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = m0 + (wm * FM + i) * 16 + g * 4 + r;
                if (row >= M)
                    continue;
                if (P)
                    P[(size_t(blockIdx.z) * M + row) * N + col] = acc[i][j][r];
                else
                    C[size_t(row) * N + col] = uint16_t(f32_to_bf16_bits(acc[i][j][r]));
            }
        }
}

template <int BM, int BN, int WM, int WN>
hipError_t launch_ctx_tile(const uint16_t *A, const uint16_t *W, uint16_t *C, float *P, int M,
                           int N, int K, CtxSplit sp, hipStream_t s)
{
    auto kern = ctx_gemm_kernel<BM, BN, WM, WN>;
    const size_t lds = size_t(2 * (BM + BN) * LDR) * 2;
    if (lds > 65536)
        (void)hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
    const dim3 grid((N + BN - 1) / BN, (M + BM - 1) / BM, sp.S);
    hipLaunchKernelGGL(kern, grid, dim3(WM * WN * 64), lds, s, A, W, C, sp.S > 1 ? P : nullptr, M,
                       N, K, sp.Ks);
    return hipGetLastError();
}

constexpr int BM = 128, BN = 128;

CtxSplit ctx_split(int M, int N, int K)
{
    const long tiles = long((N + BN - 1) / BN) * long((M + BM - 1) / BM);
    constexpr long kTarget = 512;  // two 256-thread workgroups on each of 256 CUs
    if (tiles * 4 >= kTarget * 3)
        return CtxSplit{1, K};
    int S = int((kTarget + tiles - 1) / tiles);
    // an even number of 64-column steps per split (the kernel runs them in pairs)
    int Ks = ((K + S - 1) / S + 2 * BK - 1) / (2 * BK) * (2 * BK);
    if (Ks < 4 * BK)
        Ks = 4 * BK;  // at least four K steps per split
    if (Ks > K)
        Ks = K;
    S = (K + Ks - 1) / Ks;
    return CtxSplit{S, Ks};
}

hipError_t launch_ctx_gemm(const uint16_t *A, const uint16_t *W, uint16_t *C, float *P, int M,
                           int N, int K, CtxSplit sp, hipStream_t s)
{
    return launch_ctx_tile<BM, BN, 4, 2>(A, W, C, P, M, N, K, sp, s);
}

}  // namespace mtp
