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
//   * The activations of a K-chunk are staged in LDS once per workgroup
//     ([B][KC + 8] BF16, rows padded by 16 B so the 16 lanes of a row group hit
//     distinct banks).  Lanes of padded batch rows (m >= B) read a staged row
//     too: their output rows are never read, and MFMA output rows depend only
//     on their own A row.  With
//     160 KiB of LDS a whole K = 6144 chunk fits up to B = 12.  Each wave owns
//     an equal contiguous share of the weight rows, walks the 16-row tiles that
//     cover it (MAXT per pass, accumulators kept across chunks) and loads only
//     its own rows.
//   * FP8 codes are decoded to BF16 in registers (v_cvt_scalef32_pk_bf16_fp8
//     with scale 1, exact for every E4M3FN value); the per-row scale multiplies
//     the FP32 sum once, as the FP8 head defines it.
//   * Weights stream with 16-byte non-temporal loads, 16 KiB in flight per wave.
#include "common.hpp"
#include "kernels.hpp"
#include "mfma_util.hpp"

namespace mtp {

template <bool FP8, int EPI, int NBT, int MAXT, int UK, int WPB, bool MULTI, bool RR = false>
__global__ __launch_bounds__(WPB * 64) void mfma_gemm_kernel(MfmaArgs a)
{
    extern __shared__ uint4 lds_raw[];
    uint16_t *As = reinterpret_cast<uint16_t *>(lds_raw);
    constexpr int BP = 16 * NBT;  // padded batch rows
    constexpr int NT = WPB * kWave;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    // the wave index is uniform across the wave; saying so keeps everything
    // derived from it (row range, buffer resource) in scalar registers
    const int wid = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int nl = lane & 15;  // weight row within a tile / batch row within a batch tile
    const int g = lane >> 4;   // k-slot group
    const int KC = a.KC;
    const int rs = KC + 8;     // LDS row stride in BF16 elements (16 B of padding)
    const int B = a.B;
    const int N = a.N;
    const int K = a.K;
    const int split = blockIdx.y;
    const int k_begin = split * a.Ks;
    const int k_end = min(K, k_begin + a.Ks);
    const int nchunks = (k_end - k_begin + KC - 1) / KC;
    const char *Wb = reinterpret_cast<const char *>(a.W);
    const size_t wrow = FP8 ? size_t(K) : size_t(K) * 2;  // bytes per weight row
    constexpr int ESZ = FP8 ? 1 : 2;
    // this wave's 2 KiB exchange scratch, after the staged activations
    char *xs = reinterpret_cast<char *>(lds_raw) + a.xs_off + wid * 2048;

    // Rows go to waves in one of two ways.  By default each wave owns a
    // contiguous, equal share of the rows (balanced in bytes); its tiles are
    // the 16-row blocks that overlap the share, and rows outside the share
    // are neither loaded nor reported.  With RR (the lm_head sweeps) 16-row
    // tiles are dealt round-robin to the grid's waves instead, so the grid
    // streams one window of the matrix at a time: measured 3-7% faster than
    // 2048 waves each streaming its own region.
    const int Wt = gridDim.x * WPB;
    // The wave's slot in the grid.  Tiles go to slots in order (RR), so with
    // fewer tiles than waves the slots are numbered across workgroups first:
    // every CU then gets a share instead of the first workgroups all of it.
    const int gw = (RR && a.spread) ? wid * int(gridDim.x) + int(blockIdx.x)
                                    : int(blockIdx.x) * WPB + wid;
    const int R = (N + Wt - 1) / Wt;
    int r_lo = min(N, gw * R);
    int r_hi = min(N, r_lo + R);
    const int t_lo = r_lo / 16;
    const int ntiles = r_hi > r_lo ? (r_hi + 15) / 16 - t_lo : 0;
    // The wave's rows as a buffer resource: loads outside [r_lo, r_hi) return
    // zero in hardware, so partial tiles need no per-lane predicates.
    __amdgpu_buffer_rsrc_t wrsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char *>(Wb) + size_t(r_lo) * wrow, 0, int(size_t(r_hi - r_lo) * wrow), 0x00020000);
    // With several K-chunks (MULTI): passes of MAXT tiles whose accumulators
    // live across the chunks; the same pass count in every wave of the
    // workgroup, so the barriers match.
    const int npass = ((R + 15) / 16 + 1 + MAXT - 1) / MAXT;

    // Stage the activations of one K-chunk: up to SB 16-byte loads per thread
    // are issued before any of them is stored, so the chunk costs about one
    // memory latency rather than one per load.
    auto stage = [&](int kc0) {
        constexpr int SB = NBT >= 3 ? 8 : 16;  // fewer where the batch tiles hold many registers
        const int kc_len = min(KC, k_end - kc0);
        const int n16 = B * (KC / 8);
        for (int i0 = tid; i0 < n16; i0 += SB * NT) {
            uint4 v[SB];
#pragma unroll
            for (int j = 0; j < SB; ++j) {
                const int i = i0 + j * NT;
                const int bb = i / (KC / 8);
                const int c = (i - bb * (KC / 8)) * 8;
                v[j] = make_uint4(0, 0, 0, 0);
                if (i < n16 && c < kc_len)
                    v[j] = *reinterpret_cast<const uint4 *>(a.A + size_t(bb) * K + kc0 + c);
            }
#pragma unroll
            for (int j = 0; j < SB; ++j) {
                const int i = i0 + j * NT;
                const int bb = i / (KC / 8);
                const int c = (i - bb * (KC / 8)) * 8;
                if (i < n16)
                    *reinterpret_cast<uint4 *>(As + size_t(bb) * rs + c) = v[j];
            }
        }
    };

    float best_v[NBT][4];
    uint32_t best_i[NBT][4];
#pragma unroll
    for (int bt = 0; bt < NBT; ++bt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            best_v[bt][i] = -INFINITY;
            best_i[bt][i] = 0xFFFFFFFFu;
        }

    // One group = 16 loads per lane = 8 segments of 128 B per row of a 16-row
    // tile (BF16: 16 k-steps; FP8: 16 step pairs).  Load 2j fetches tile rows
    // 0-7, load 2j+1 rows 8-15 of segment j, 8 lanes x 16 B per row, so every
    // load instruction reads whole 128-B lines.
    constexpr int NL = 16;
    static_assert((FP8 ? UK / 2 : UK) == NL, "one group = 8 segments");
    auto load_group = [&](uint4 (&raw)[NL], int tile0, int s0, int kc0, int kc_len) {
        const int seg0 = kc0 * ESZ + (FP8 ? (s0 >> 1) * 64 : s0 * 64);  // row byte offset
        const int lim = (kc0 + kc_len) * ESZ;  // end of this chunk in the row
        // byte offsets inside the wave's rows; rows below r_lo go negative,
        // i.e. huge as unsigned, and rows at or past r_hi exceed the range
        const int vo0 = (tile0 - r_lo + (lane >> 3)) * int(wrow) + seg0 + (lane & 7) * 16;
        const int vo1 = vo0 + 8 * int(wrow);
        if (seg0 + 1024 <= lim) {
#pragma unroll
            for (int u = 0; u < NL; ++u)
                raw[u] = ld_buf16(wrsrc, ((u & 1) ? vo1 : vo0) + (u >> 1) * 128);
        } else {
            // last group of a chunk: columns past the chunk read as zero too
#pragma unroll
            for (int u = 0; u < NL; ++u) {
                const bool col_ok = seg0 + (u >> 1) * 128 + (lane & 7) * 16 < lim;
                const int vo = ((u & 1) ? vo1 : vo0) + (u >> 1) * 128;
                raw[u] = ld_buf16(wrsrc, col_ok ? vo : int(0x80000000u));
            }
        }
    };
    // Re-lay each segment through this wave's LDS scratch into MFMA layout:
    // lane (g, n) takes row n, 16-byte piece 4s + g for the segment's step
    // (pair) s = 0, 1 -- the same columns as the activation reads.  Piece p of
    // row r sits at slot p ^ ((r >> 1) & 7) so 16 lanes of a read hit distinct
    // banks.  Then one MFMA per k-step and batch tile.
    auto compute_group = [&](uint4 (&raw)[NL], f32x4 (&acc)[NBT], int s0, int nsteps) {
#pragma unroll
        for (int j = 0; j < NL / 2; ++j) {
            const int wr0 = lane >> 3, wp = lane & 7;
            *reinterpret_cast<uint4 *>(xs + wr0 * 128 + ((wp ^ ((wr0 >> 1) & 7)) * 16)) = raw[2 * j];
            const int wr1 = 8 + wr0;
            *reinterpret_cast<uint4 *>(xs + wr1 * 128 + ((wp ^ ((wr1 >> 1) & 7)) * 16)) = raw[2 * j + 1];
            raw[2 * j] = *reinterpret_cast<const uint4 *>(xs + nl * 128 + ((g ^ ((nl >> 1) & 7)) * 16));
            raw[2 * j + 1] =
                *reinterpret_cast<const uint4 *>(xs + nl * 128 + (((4 + g) ^ ((nl >> 1) & 7)) * 16));
        }
        // Every k-step of the group runs: a step past the chunk has zero
        // weights (their loads read past the resource) and reads staged
        // column 0 (finite), so it adds exactly zero.  No per-step branch, so
        // the compiler can issue the activation reads ahead of the MFMAs
        // instead of waiting for each one in turn.
#pragma unroll
        for (int u = 0; u < UK; ++u) {
            bf16x8 wf;
            if (FP8) {
                const uint4 &r = raw[u >> 1];
                wf = (u & 1) ? fp8x8_to_bf16(r.z, r.w) : fp8x8_to_bf16(r.x, r.y);
            } else {
                wf = as_bf16x8(raw[u]);
            }
            const int st = s0 + u;
            const int lc = st >= nsteps ? 0
                           : FP8        ? (st >> 1) * 64 + g * 16 + (st & 1) * 8
                                        : st * 32 + g * 8;
#pragma unroll
            for (int bt = 0; bt < NBT; ++bt) {
                // padded batch rows only feed output rows that are dropped,
                // so they may read any staged row
                const int arow = min(bt * 16 + nl, B - 1);
                const uint4 av = *reinterpret_cast<const uint4 *>(As + size_t(arow) * rs + lc);
                acc[bt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(av), wf, acc[bt], 0, 0,
                                                                  0);
            }
        }
    };
    // Rows of one finished tile: store / round, argmax bookkeeping.
    auto epilogue = [&](f32x4 (&acc)[NBT], int tile0) {
        const int row = tile0 + nl;
        if (row < r_lo || row >= r_hi)
            return;
        const float sc = (FP8 && EPI == EPI_ARGMAX) ? a.scale[row] : 1.0f;
#pragma unroll
        for (int bt = 0; bt < NBT; ++bt) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int bb = bt * 16 + g * 4 + i;
                if (bb >= B)
                    continue;
                const float z = acc[bt][i];
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
    };

    if (!MULTI) {
        // One chunk holds all of K: walk the tiles one by one with a single
        // accumulator.  (Double-buffering the groups in registers was measured:
        // no gain for the head, and the extra registers cost the split-K
        // eh_proj a workgroup per CU.)
        const int kc_len = k_end - k_begin;
        const int nsteps = FP8 ? 2 * ((kc_len + 63) / 64) : (kc_len + 31) / 32;
        // RR: 16-row tiles dealt round-robin to the grid's waves, so the grid
        // sweeps one window of the matrix at a time; each tile its own
        // resource (rows past N read zero)
        const int t_first = RR ? gw : t_lo;
        const int t_stop = RR ? (N + 15) / 16 : t_lo + ntiles;
        const int t_step = RR ? Wt : 1;
        auto set_tile = [&](int tile0) {
            if constexpr (RR) {
                // a tile at or past N (a wave with no tile) gets an empty range
                r_lo = min(N, tile0);
                r_hi = min(N, tile0 + 16);
                wrsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(Wb) + size_t(r_lo) * wrow,
                                                          0, int(size_t(r_hi - r_lo) * wrow), 0x00020000);
            }
        };
        // eh_proj (three groups per wave): the first group's weight loads go
        // out before the activations are staged, so the two latencies overlap
        // (measured 4 us off the B = 16 sweep).  The long head sweeps measured
        // 1% slower with it and skip it.  A wave with no tile loads through an
        // empty or zero-length range: zeros, no memory access.
        constexpr bool PRE = EPI == EPI_STORE;
        uint4 raw[NL];
        if constexpr (PRE) {
            set_tile(t_first * 16);
            load_group(raw, t_first * 16, 0, k_begin, kc_len);
        }
        stage(k_begin);
        __syncthreads();
        bool have = PRE;
#pragma unroll 1
        for (int t = t_first; t < t_stop; t += t_step) {
            const int tile0 = t * 16;
            set_tile(tile0);
            f32x4 acc[NBT];
#pragma unroll
            for (int bt = 0; bt < NBT; ++bt)
                acc[bt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 1
            for (int s0 = 0; s0 < nsteps; s0 += UK) {
                if (!PRE || !have)
                    load_group(raw, tile0, s0, k_begin, kc_len);
                have = false;
                compute_group(raw, acc, s0, nsteps);
            }
            epilogue(acc, tile0);
        }
    } else {
        // RR as above; the pass count stays the same in every wave of the
        // workgroup (the chunk barriers), each tile's resource is made again
        // before its loads and its epilogue
        const int T16 = (N + 15) / 16;
        const int nt_w = RR ? (gw < T16 ? (T16 - gw + Wt - 1) / Wt : 0) : ntiles;
        const int npass_w = RR ? ((T16 + Wt - 1) / Wt + MAXT - 1) / MAXT : npass;
        auto tile_of = [&](int tix) { return RR ? (gw + tix * Wt) * 16 : (t_lo + tix) * 16; };
        auto set_tile = [&](int tile0) {
            if constexpr (RR) {
                // a tile at or past N (a wave with no tile) gets an empty range
                r_lo = min(N, tile0);
                r_hi = min(N, tile0 + 16);
                wrsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(Wb) + size_t(r_lo) * wrow,
                                                          0, int(size_t(r_hi - r_lo) * wrow), 0x00020000);
            }
        };
#pragma unroll 1
        for (int pass = 0; pass < npass_w; ++pass) {
            f32x4 acc[MAXT][NBT];
#pragma unroll
            for (int j = 0; j < MAXT; ++j)
#pragma unroll
                for (int bt = 0; bt < NBT; ++bt)
                    acc[j][bt] = f32x4{0.f, 0.f, 0.f, 0.f};
            for (int ch = 0; ch < nchunks; ++ch) {
                const int kc0 = k_begin + ch * KC;
                const int kc_len = min(KC, k_end - kc0);  // a multiple of 16
                // k-steps of 32 columns.  FP8 loads cover a pair of steps (64
                // columns), so the FP8 count is a whole number of pairs; columns
                // past the chunk are zero in LDS and not loaded from HBM.
                const int nsteps = FP8 ? 2 * ((kc_len + 63) / 64) : (kc_len + 31) / 32;
                __syncthreads();  // the previous chunk's LDS reads are done
                // the pass's first group goes out with the staging loads
                uint4 raw[NL];
                const bool pre = pass * MAXT < nt_w;
                if (pre) {
                    set_tile(tile_of(pass * MAXT));
                    load_group(raw, tile_of(pass * MAXT), 0, kc0, kc_len);
                }
                stage(kc0);
                __syncthreads();
                bool have = pre;
#pragma unroll
                for (int j = 0; j < MAXT; ++j) {
                    const int tix = pass * MAXT + j;
                    if (tix >= nt_w)
                        continue;  // uniform across the wave
                    const int tile0 = tile_of(tix);
                    set_tile(tile0);
#pragma unroll 1
                    for (int s0 = 0; s0 < nsteps; s0 += UK) {
                        if (!have)
                            load_group(raw, tile0, s0, kc0, kc_len);
                        have = false;
                        compute_group(raw, acc[j], s0, nsteps);
                    }
                }
            }
#pragma unroll
            for (int j = 0; j < MAXT; ++j) {
                const int tix = pass * MAXT + j;
                if (tix < nt_w) {
                    set_tile(tile_of(tix));
                    epilogue(acc[j], tile_of(tix));
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
        uint32_t *ri = reinterpret_cast<uint32_t *>(rv + WPB * BP);
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
        for (int bb = tid; bb < B; bb += NT) {
            float bv = rv[bb];
            uint32_t bi = ri[bb];
            for (int w = 1; w < WPB; ++w)
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

// Per-workgroup LDS bytes the current device allows (160 KiB on gfx950).
static int lds_limit()
{
    int dev = 0, v = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) == hipSuccess &&
        v > 0)
        return v;
    return 65536;
}

// Chunk width: the largest multiple of 64 whose [B][KC + 8] BF16 tile fits
// the LDS budget, then evened out over the chunks a split needs.
static int chunk_cols(int B, int klen, int wpb)
{
    const int budget = min(lds_limit(), 160 * 1024) - 2048 - wpb * 2048;
    int kc_max = (budget / (B * 2) - 8) / 64 * 64;
    if (kc_max < 64)
        kc_max = 64;
    const int nch = (klen + kc_max - 1) / kc_max;
    int kc = ((klen + nch - 1) / nch + 63) / 64 * 64;
    return kc < 64 ? 64 : kc;
}

template <bool FP8, int EPI, int NBT, int WPB>
static hipError_t launch_mfma_nbt(MfmaArgs a, int grid, int splits, hipStream_t s)
{
    // Tiles per pass with several K-chunks: every pass restages the chunks,
    // so one pass should cover a wave's tiles.  The Large lm_head deals ~5
    // tiles to each of 2048 waves; 6 keeps B <= 16 to one pass (measured 2%
    // faster than 4 at B = 16 FP8) without spilling.  The split-K eh_proj
    // runs 3 workgroups per CU and keeps 4 (fewer registers).
    constexpr int MAXT = NBT == 1 ? (EPI == EPI_ARGMAX ? 6 : 4) : (NBT == 2 ? 2 : 1);
    constexpr int UK = FP8 ? 32 : 16;
    a.KC = chunk_cols(a.B, a.Ks, WPB);
    const bool multi = a.KC < a.Ks;
    auto kern = multi ? mfma_gemm_kernel<FP8, EPI, NBT, MAXT, UK, WPB, true, EPI == EPI_ARGMAX>
                      : mfma_gemm_kernel<FP8, EPI, NBT, 1, UK, WPB, false, EPI == EPI_ARGMAX>;
    a.xs_off = int(align256(size_t(a.B) * size_t(a.KC + 8) * 2));
    size_t lds = size_t(a.xs_off) + size_t(WPB) * 2048;
    const size_t red = size_t(WPB * 16 * NBT) * 8;
    if (lds < red)
        lds = red;
    if (lds > 65536)
        (void)hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
    hipLaunchKernelGGL(kern, dim3(grid, splits), dim3(WPB * 64), lds, s, a);
    return hipGetLastError();
}

template <bool FP8, int EPI, int WPB>
static hipError_t launch_mfma(const MfmaArgs &a, int grid, int splits, hipStream_t s)
{
    switch ((a.B + 15) / 16) {
    case 1: return launch_mfma_nbt<FP8, EPI, 1, WPB>(a, grid, splits, s);
    case 2: return launch_mfma_nbt<FP8, EPI, 2, WPB>(a, grid, splits, s);
    case 3: return launch_mfma_nbt<FP8, EPI, 3, WPB>(a, grid, splits, s);
    default: return launch_mfma_nbt<FP8, EPI, 4, WPB>(a, grid, splits, s);
    }
}

// eh_proj (N = H rows, K = 2H) for B >= 2: one 16-row tile per wave, four
// waves per workgroup, K split so that the grid is about 3 workgroups per CU.
EhSplit eh_split(int hidden)
{
    const int T = (hidden + 15) / 16;
    const int K = 2 * hidden;
    const int wgs_per_split = (T + 3) / 4;
    int S = (768 + wgs_per_split - 1) / wgs_per_split;
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
    return launch_mfma<false, EPI_STORE, 4>(a, grid, sp.S, s);
}

// lm_head for B >= 2: one 8-wave workgroup per CU sharing the staged
// activations; 16-row tiles dealt round-robin to the grid's waves.  Every CU
// gets a workgroup as long as there is a tile for each (a vocabulary shard of
// V/8 rows is 1210 tiles: 256 workgroups of 4-5 busy waves, where a floor of
// 64 rows per wave had left 38 workgroups streaming it).
hipError_t launch_head_mfma(const MfmaArgs &a_in, bool fp8, int *grid_out, hipStream_t s)
{
    if (head_tile_fits(a_in.B, a_in.K, fp8))
        return launch_head_tile(a_in, fp8, grid_out, s);
    MfmaArgs a = a_in;
    a.Ks = a.K;
    const int tiles = (a.N + 15) / 16;
    int grid = device_cu_count();
    if (grid > tiles)
        grid = tiles;
    if (grid > kMaxHeadBlocks)
        grid = kMaxHeadBlocks;
    if (grid < 1)
        grid = 1;
    a.spread = tiles < grid * 8;
    *grid_out = grid;
    return fp8 ? launch_mfma<true, EPI_ARGMAX, 8>(a, grid, 1, s)
               : launch_mfma<false, EPI_ARGMAX, 8>(a, grid, 1, s);
}

}  // namespace mtp
