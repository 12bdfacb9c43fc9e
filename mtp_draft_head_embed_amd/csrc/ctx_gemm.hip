// ctx_gemm.hip -- the drafter's context rows (metrale_model_arch/
// glm5next_mtp_head.rs, `rows_impl`): T prompt or catch-up rows through the
// front half, row r pairing embed(tokens[r + 1]) with hiddens[r]:
//
//   x[r] = BF16(eh_proj . [enorm(embed[tokens[r+1]]) | hnorm(hiddens[r])])
//
// The page stops each row at the block's KV-cache write (out of scope here).
// With T rows, eh_proj is a dense GEMM C[T][H] = A[T][2H] . W[H][2H]^T with
// both operands K-contiguous, HBM-bound for a few hundred rows and bound by
// the matrix cores beyond.  One kernel, three tile shapes:
//   * 256 x 256 or 256 x 192 output tile per 16-wave workgroup (one per CU)
//     for many rows (whichever fills the CUs in whole rounds; the 192-wide
//     tile on 8 waves when its grid is whole rounds), 128 x 128 per 8-wave
//     workgroup up to 128 rows; every wave owns a 64 x 64, 64 x 96, 64 x 48
//     or 64 x 32 block of v_mfma_f32_16x16x32_bf16 accumulators;
//   * K in steps of 64 columns (128-byte staged rows, 8 rows per load
//     instruction) through LDS stages, each its own LDS object; the operands
//     go from HBM straight into LDS (buffer loads with the LDS flag: no
//     registers, no LDS store instructions).  The skinny tile keeps four
//     stages, its loads issued three steps ahead (its time goes to streaming
//     eh_proj, 128 contiguous bytes of a weight row per load); the large
//     tiles fit two stages of 64 columns, the next step's loads issued while
//     a step computes: half the barriers of 32-column steps through four
//     stages, measured 1.5-4.4% faster from T = 1024 to 16 384 (a step is long
//     enough for its mostly L2-resident loads to land);
//   * 16-byte piece c of staged row r sits at slot c ^ ((r >> 1) & (n - 1))
//     for n pieces per row, so the 16-lane fragment reads hit distinct banks;
//   * the fragment reads are plain ds_read_b128 the compiler does not see as
//     LDS accesses, with explicit waits that the MFMAs depend on: otherwise
//     it waits for every load in flight before each read (it cannot tell
//     that they fill other stages), and a fenced barrier would do the same;
//   * on 64-column steps the second 32-column sub-step's A fragments are read
//     into each register as soon as the first sub-step's MFMAs that use it
//     have issued, so only the W fragment reads are waited for in full;
//   * a wave raises its priority while it issues its MFMAs, so the SIMD's
//     arbiter prefers waves with matrix work ready over waves that are about
//     to read LDS or wait (1-2% faster from T = 1024 to 16 384);
//   * rows past T or H and columns past the split read zero (the buffer
//     resource's range; an offset past it);
//   * with few tiles (a skinny T) K is split over blockIdx.z so that the
//     CUs are filled; each split writes an FP32 partial tile and the splits
//     are summed in split order by the batched path's sum-and-round kernel.
// Sums are FP32 in a fixed k order, the same for every tile shape, so results
// depend neither on timing nor on the shape chosen.
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"
#include "ctx_gemm.hpp"

namespace mtp {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;

// Slot of 16-byte piece `piece` of staged row `row` when a staged row holds
// NP pieces (NP = 4: 64 bytes, 32 columns; NP = 8: 128 bytes, 64 columns):
// rows of the same parity start at the same bank, and the XOR spreads the
// 16 rows of a fragment read over distinct 16-byte bank groups.
template <int NP>
__host__ __device__ __forceinline__ int slot(int row, int piece)
{
    return piece ^ ((row >> 1) & (NP - 1));
}

__device__ __forceinline__ bf16x8_t as_bf16x8(const u32x4_t &u)
{
    return __builtin_bit_cast(bf16x8_t, u);
}

// LDS byte offset of a __shared__ object (its flat address keeps the offset
// in the low 32 bits)
__device__ __forceinline__ uint32_t lds_offset(const void *p)
{
    return uint32_t(reinterpret_cast<uintptr_t>(p));
}

}  // namespace

template <int BM, int BN, int WM, int WN, int BK = 32, int NST = 4, bool PREFETCH_A = true>
__global__ __launch_bounds__(WM *WN * 64) void ctx_gemm_kernel(const uint16_t *__restrict__ A,
                                                               const uint16_t *__restrict__ W,
                                                               uint16_t *__restrict__ C,
                                                               float *__restrict__ P, int M, int N,
                                                               int K, int Ks)
{
    // BK columns per step: each staged row holds RB = 2 BK bytes in NP pieces
    // of 16, and one load instruction stages RPL = 64 / NP rows
    static_assert(BK == 32 || BK == 64, "steps of 32 or 64 columns");
    constexpr int RB = BK * 2, NP = RB / 16, RPL = 64 / NP, NSUB = BK / 32;
    constexpr int NW = WM * WN;
    constexpr int FM = BM / WM / 16, FN = BN / WN / 16;
    static_assert(FM == 4, "the staged waits below assume four A fragments per wave");
    static_assert((FN >= 2 && FN <= 4) || FN == 6, "two to four, or six, W fragments per wave");
    // A load instruction stages RPL rows (16 of 64 bytes or 8 of 128).  The A
    // rows go to the waves in equal contiguous shares of whole load
    // instructions; so do the W rows when they divide so (192 rows over 8
    // waves: 24 each), else W row group q (16 rows) goes to wave q, and the
    // waves past the last group stage nothing real: their load reads past the
    // resource (zeros) into a slot of 16 staged rows past the stage, so every
    // wave issues the same number of loads per step and the vmcnt waits below
    // hold for all of them.
    constexpr int RA = BM / NW;
    static_assert(RA % RPL == 0 && BN % 16 == 0, "waves stage whole load instructions");
    constexpr bool WSPLIT = (BN / NW) % RPL == 0;
    static_assert(WSPLIT || BN / 16 <= NW, "uneven W staging takes one group per wave");
    constexpr int RW = WSPLIT ? BN / NW : 16;
    constexpr int IA = RA / RPL, IW = RW / RPL;
    constexpr int STAGE = (BM + BN) * RB + (WSPLIT ? 0 : (NW - BN / 16) * 16 * RB);
    // NST stages, loads issued NST - 1 steps ahead: the NST - 2 newer stages
    // may stay in flight when a step's stage must be in
    static_assert(NST >= 2 && NST <= 4, "two to four stages");
    constexpr int INFLIGHT = (NST - 2) * (IA + IW);
    __shared__ __attribute__((aligned(1024))) char st0[STAGE];
    __shared__ __attribute__((aligned(1024))) char st1[STAGE];
    __shared__ __attribute__((aligned(1024))) char st2[NST > 2 ? STAGE : 16];
    __shared__ __attribute__((aligned(1024))) char st3[NST > 3 ? STAGE : 16];
    auto stage = [&](auto sc) -> char * {
        constexpr int S = decltype(sc)::value;
        if constexpr (S == 0)
            return st0;
        else if constexpr (S == 1)
            return st1;
        else if constexpr (S == 2)
            return st2;
        else
            return st3;
    };

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wid / WN, wn = wid % WN;
    const int nl = lane & 15, g = lane >> 4;
    const int m0 = blockIdx.y * BM;
    const int n0 = blockIdx.x * BN;
    const int k_begin = blockIdx.z * Ks;
    const int k_end = min(K, k_begin + Ks);
    const uint32_t rowb = uint32_t(K) * 2;

    // The tile's rows as buffer resources: rows past M (N) read as zero.
    const __amdgpu_buffer_rsrc_t arsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(A) + size_t(m0) * K, 0, int(uint32_t(min(BM, M - m0)) * rowb),
        0x00020000);
    const __amdgpu_buffer_rsrc_t wrsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(W) + size_t(n0) * K, 0, int(uint32_t(min(BN, N - n0)) * rowb),
        0x00020000);
    // A load instruction stages RPL rows from row r0 on: lane L takes row
    // r0 + L / NP and LDS slot L % NP, which holds piece slot<NP>(row, L % NP)
    // of the row's RB bytes (the XOR is its own inverse, and it depends on
    // the row within its 16-row group, as the fragment reads below do).
    const int lrow = lane / NP, lslot = lane % NP;
    // A piece past the split reads zero (an offset past the range): K and
    // the split bounds are multiples of 32 columns, so a 64-column step can
    // end half past the split, and must not read the next row's first columns.
    auto issue = [&](char *st, int k0) {
#pragma unroll
        for (int j = 0; j < IA + IW; ++j) {
            const bool is_a = j < IA;
            const int r0 = is_a ? wid * RA + RPL * j : wid * RW + RPL * (j - IA);
            const int pc = slot<NP>(r0 + lrow, lslot);
            // uneven W staging: a wave past the last group fills its own slot
            // after the stage's W rows with zeros (an offset past the range)
            const bool live = k0 + pc * 8 < k_end && (is_a || WSPLIT || r0 < BN);
            const uint32_t off = live ? uint32_t(r0 + lrow) * rowb + uint32_t(pc) * 16 +
                                            uint32_t(k0) * 2
                                      : 0x80000000u;
            char *dst = is_a ? st + r0 * RB : st + BM * RB + r0 * RB;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(is_a ? arsrc : wrsrc, (lds_void_t *)dst, 16,
                                                     off, 0, 0, 0);
        }
    };

    // fragment addresses inside a stage: for the 32 columns of sub-step u,
    // lane (g, n) reads row n, piece 4u + g
    uint32_t aoff[NSUB][FM], woff[NSUB][FN];
#pragma unroll
    for (int u = 0; u < NSUB; ++u) {
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const int row = (wm * FM + i) * 16 + nl;
            aoff[u][i] = uint32_t(row * RB + slot<NP>(row, 4 * u + g) * 16);
        }
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int row = (wn * FN + j) * 16 + nl;
            woff[u][j] = uint32_t(BM * RB + row * RB + slot<NP>(row, 4 * u + g) * 16);
        }
    }

    f32x4_t acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
            acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    auto mma_row = [&](auto ic, const u32x4_t &a, const u32x4_t(&w)[FN]) {
        constexpr int i = decltype(ic)::value;
#pragma unroll
        for (int j = 0; j < FN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(w[j]),
                                                                acc[i][j], 0, 0, 0);
    };
    // one sub-step: 32 columns of the stage, in k order
    auto compute_sub = [&](const char *st, const uint32_t(&ao)[FM], const uint32_t(&wo)[FN]) {
        const uint32_t base = lds_offset(st);
        u32x4_t a[FM], w[FN];
#pragma unroll
        for (int j = 0; j < FN; ++j)
            asm volatile("ds_read_b128 %0, %1" : "=v"(w[j]) : "v"(base + wo[j]));
#pragma unroll
        for (int i = 0; i < FM; ++i)
            asm volatile("ds_read_b128 %0, %1" : "=v"(a[i]) : "v"(base + ao[i]));
        // W and A row i are in once at most 3 - i reads are outstanding
        if constexpr (FN == 6)
            asm volatile("s_waitcnt lgkmcnt(3)"
                         : "+v"(a[0]), "+v"(w[0]), "+v"(w[1]), "+v"(w[2]), "+v"(w[3]), "+v"(w[4]),
                           "+v"(w[5]));
        else if constexpr (FN == 4)
            asm volatile("s_waitcnt lgkmcnt(3)"
                         : "+v"(a[0]), "+v"(w[0]), "+v"(w[1]), "+v"(w[2]), "+v"(w[3]));
        else if constexpr (FN == 3)
            asm volatile("s_waitcnt lgkmcnt(3)" : "+v"(a[0]), "+v"(w[0]), "+v"(w[1]), "+v"(w[2]));
        else
            asm volatile("s_waitcnt lgkmcnt(3)" : "+v"(a[0]), "+v"(w[0]), "+v"(w[1]));
        __builtin_amdgcn_s_setprio(1);
        mma_row(std::integral_constant<int, 0>{}, a[0], w);
        asm volatile("s_waitcnt lgkmcnt(2)" : "+v"(a[1]));
        mma_row(std::integral_constant<int, 1>{}, a[1], w);
        asm volatile("s_waitcnt lgkmcnt(1)" : "+v"(a[2]));
        mma_row(std::integral_constant<int, 2>{}, a[2], w);
        asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(a[3]));
        mma_row(std::integral_constant<int, 3>{}, a[3], w);
        __builtin_amdgcn_s_setprio(0);
    };
    // Two sub-steps: the second's A fragment i is read into a[i] as soon as
    // the first's row i has issued its MFMAs (no extra registers), so those
    // reads overlap the first sub-step's matrix work; only the second's W
    // fragments wait in full.
    auto compute2 = [&](const char *st) {
        const uint32_t base = lds_offset(st);
        u32x4_t a[FM], w[FN];
#pragma unroll
        for (int j = 0; j < FN; ++j)
            asm volatile("ds_read_b128 %0, %1" : "=v"(w[j]) : "v"(base + woff[0][j]));
#pragma unroll
        for (int i = 0; i < FM; ++i)
            asm volatile("ds_read_b128 %0, %1" : "=v"(a[i]) : "v"(base + aoff[0][i]));
        if constexpr (FN == 6)
            asm volatile("s_waitcnt lgkmcnt(3)"
                         : "+v"(a[0]), "+v"(w[0]), "+v"(w[1]), "+v"(w[2]), "+v"(w[3]), "+v"(w[4]),
                           "+v"(w[5]));
        else if constexpr (FN == 4)
            asm volatile("s_waitcnt lgkmcnt(3)"
                         : "+v"(a[0]), "+v"(w[0]), "+v"(w[1]), "+v"(w[2]), "+v"(w[3]));
        else if constexpr (FN == 3)
            asm volatile("s_waitcnt lgkmcnt(3)" : "+v"(a[0]), "+v"(w[0]), "+v"(w[1]), "+v"(w[2]));
        else
            asm volatile("s_waitcnt lgkmcnt(3)" : "+v"(a[0]), "+v"(w[0]), "+v"(w[1]));
        __builtin_amdgcn_s_setprio(1);
        // in flight before each row: the first sub-step's rows i..3 and the
        // second's rows 0..i-1; reads complete in issue order
        mma_row(std::integral_constant<int, 0>{}, a[0], w);
        asm volatile("ds_read_b128 %0, %2\n\ts_waitcnt lgkmcnt(3)"
                     : "=v"(a[0]), "+v"(a[1]) : "v"(base + aoff[1][0]));
        mma_row(std::integral_constant<int, 1>{}, a[1], w);
        asm volatile("ds_read_b128 %0, %2\n\ts_waitcnt lgkmcnt(3)"
                     : "=v"(a[1]), "+v"(a[2]) : "v"(base + aoff[1][1]));
        mma_row(std::integral_constant<int, 2>{}, a[2], w);
        asm volatile("ds_read_b128 %0, %2\n\ts_waitcnt lgkmcnt(3)"
                     : "=v"(a[2]), "+v"(a[3]) : "v"(base + aoff[1][2]));
        mma_row(std::integral_constant<int, 3>{}, a[3], w);
        asm volatile("ds_read_b128 %0, %1" : "=v"(a[3]) : "v"(base + aoff[1][3]));
        __builtin_amdgcn_s_setprio(0);
#pragma unroll
        for (int j = 0; j < FN; ++j)
            asm volatile("ds_read_b128 %0, %1" : "=v"(w[j]) : "v"(base + woff[1][j]));
        if constexpr (FN == 6)
            asm volatile("s_waitcnt lgkmcnt(0)"
                         : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]), "+v"(w[0]), "+v"(w[1]),
                           "+v"(w[2]), "+v"(w[3]), "+v"(w[4]), "+v"(w[5]));
        else if constexpr (FN == 4)
            asm volatile("s_waitcnt lgkmcnt(0)"
                         : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]), "+v"(w[0]), "+v"(w[1]),
                           "+v"(w[2]), "+v"(w[3]));
        else if constexpr (FN == 3)
            asm volatile("s_waitcnt lgkmcnt(0)"
                         : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]), "+v"(w[0]), "+v"(w[1]),
                           "+v"(w[2]));
        else
            asm volatile("s_waitcnt lgkmcnt(0)"
                         : "+v"(a[0]), "+v"(a[1]), "+v"(a[2]), "+v"(a[3]), "+v"(w[0]), "+v"(w[1]));
        __builtin_amdgcn_s_setprio(1);
        mma_row(std::integral_constant<int, 0>{}, a[0], w);
        mma_row(std::integral_constant<int, 1>{}, a[1], w);
        mma_row(std::integral_constant<int, 2>{}, a[2], w);
        mma_row(std::integral_constant<int, 3>{}, a[3], w);
        __builtin_amdgcn_s_setprio(0);
    };
    auto compute = [&](const char *st) {
        if constexpr (NSUB == 2 && PREFETCH_A) {
            compute2(st);
        } else {
#pragma unroll
            for (int u = 0; u < NSUB; ++u)
                compute_sub(st, aoff[u], woff[u]);
        }
    };

    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    using I3 = std::integral_constant<int, 3>;
    // Step t uses stage t % NST; its loads were issued NST - 1 steps earlier.
    // The barrier after a step (no fence: the newer stages stay in flight)
    // makes stage t + 1 visible to every wave and frees stage t for step
    // t + NST.
    const int nk = (k_end - k_begin + BK - 1) / BK;
    issue(stage(I0{}), k_begin);
    if constexpr (NST > 2)
        issue(stage(I1{}), k_begin + BK);
    if constexpr (NST > 3)
        issue(stage(I2{}), k_begin + 2 * BK);
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(INFLIGHT) : "memory");
    auto step = [&](int t, auto cur, auto ahead) {
        issue(stage(ahead), k_begin + (t + NST - 1) * BK);
        compute(stage(cur));
        asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(INFLIGHT) : "memory");
    };
    // steps in groups of NST; a count that is not a multiple of NST runs up to
    // NST - 1 steps past the split, which read zeros and leave the sums
    // unchanged (the accumulators start at +0)
#pragma unroll 1
    for (int t = 0; t < nk; t += NST) {
        if constexpr (NST == 4) {
            step(t, I0{}, I3{});
            step(t + 1, I1{}, I0{});
            step(t + 2, I2{}, I1{});
            step(t + 3, I3{}, I2{});
        } else if constexpr (NST == 3) {
            step(t, I0{}, I2{});
            step(t + 1, I1{}, I0{});
            step(t + 2, I2{}, I1{});
        } else {
            step(t, I0{}, I1{});
            step(t + 1, I1{}, I0{});
        }
    }
    // every load has landed before the workgroup's LDS is released
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

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

template <int BM, int BN, int WM, int WN, int BK = 32, int NST = 4>
hipError_t launch_ctx_tile(const uint16_t *A, const uint16_t *W, uint16_t *C, float *P, int M,
                           int N, int K, CtxSplit sp, hipStream_t s)
{
    const dim3 grid((N + BN - 1) / BN, (M + BM - 1) / BM, sp.S);
    hipLaunchKernelGGL((ctx_gemm_kernel<BM, BN, WM, WN, BK, NST>), grid, dim3(WM * WN * 64), 0, s,
                       A, W, C, sp.S > 1 ? P : nullptr, M, N, K, sp.Ks);
    return hipGetLastError();
}

// K split of one tile shape: at most `target` workgroups (256, one per CU),
// all in one round.
static CtxSplit split_for(int M, int N, int K, int tile, int tm, int tn, long target)
{
    const long tiles = long((N + tn - 1) / tn) * long((M + tm - 1) / tm);
    if (tiles * 4 >= target * 3)
        return CtxSplit{1, K, tile};
    // the most splits whose workgroups all run at once: one more leaves a
    // second, nearly empty round of workgroups
    int S = int(target / tiles);
    if (S < 1)
        S = 1;
    // a multiple of 128 columns per split, at least four steps
    int Ks = ((K + S - 1) / S + 127) / 128 * 128;
    if (Ks > K)
        Ks = K;
    S = (K + Ks - 1) / Ks;
    return CtxSplit{S, Ks, tile};
}

CtxSplit ctx_split(int M, int N, int K)
{
    // the skinny tile stages 64 columns per step (128 KiB of LDS: one
    // workgroup per CU); from 17 to 64 rows half its A rows are past T and
    // read zero, and it still streams eh_proj faster than a 64 x 256 tile
    // (160 KiB per 4-wave workgroup) did
    if (M < kCtxBigTileMinRows)
        return split_for(M, N, K, kCtxTile128x128, 128, 128, 256);
    // 256 x 256 or 256 x 192, whichever finishes in less tile work: rounds
    // of 256 workgroups times the work of one workgroup (at H = 6144 the
    // 192-wide tile turns 192 or 384 workgroups into whole rounds of 256 or
    // 512)
    const CtxSplit a = split_for(M, N, K, kCtxTile256x256, 256, 256, 256);
    const CtxSplit b = split_for(M, N, K, kCtxTile256x192, 256, 192, 256);
    auto work = [&](const CtxSplit &c, int tn) {
        const long wgs = long((N + tn - 1) / tn) * long((M + 255) / 256) * c.S;
        return ((wgs + 255) / 256) * long(c.Ks) * tn;
    };
    return work(b, 192) < work(a, 256) ? b : a;
}

hipError_t launch_ctx_gemm(const uint16_t *A, const uint16_t *W, uint16_t *C, float *P, int M,
                           int N, int K, CtxSplit sp, hipStream_t s)
{
    switch (sp.tile) {
    case kCtxTile256x256:
        return launch_ctx_tile<256, 256, 4, 4, 64, 2>(A, W, C, P, M, N, K, sp, s);
    case kCtxTile256x192: {
        // 8 waves of 64 x 96 when the grid fills whole rounds of one
        // workgroup per CU (a third fewer fragment reads from LDS per flop
        // than 16 waves of 64 x 48: T = 4096 3% faster, T = 1024 and 2048
        // level); 16 waves when the last round is part-filled (T = 3072: 2%
        // faster than 8)
        const long wgs = long((N + 191) / 192) * long((M + 255) / 256) * sp.S;
        if (wgs % device_cu_count() == 0)
            return launch_ctx_tile<256, 192, 4, 2, 64, 2>(A, W, C, P, M, N, K, sp, s);
        return launch_ctx_tile<256, 192, 4, 4, 64, 2>(A, W, C, P, M, N, K, sp, s);
    }
    default:
        return launch_ctx_tile<128, 128, 2, 4, 64>(A, W, C, P, M, N, K, sp, s);
    }
}

}  // namespace mtp
