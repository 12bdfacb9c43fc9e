// row_gemv.hip -- bandwidth-bound GEMV over row-major weights, one wavefront
// per output row, for the single-sequence draft sweep on gfx950.
//
// Covers these steps of `forward_one` (metrale_model_arch/glm5next_mtp_head.rs):
//   * eh_proj:  x = BF16(eh_proj . [enorm(embed[token]) | hnorm(hidden)]).
//     The embedding-row gather and both vanilla norms run as this kernel's
//     prologue (each workgroup rebuilds the [2H] concat in LDS), so there are
//     no separate norm launches.
//   * lm_head, BF16 (`dense_gemv`) and FP8 (`dense_gemv_fp8w`), with the
//     `shared_head.norm` of x as the prologue (the normed BF16 vector staged in
//     LDS) and the first argmax stage (`argmax_bf16`) as the epilogue: every
//     logit is rounded to BF16 and optionally stored (staged per wave in LDS,
//     written in batches), and each workgroup leaves
//     its best (value, index) in a partials array; argmax_final_kernel, one
//     wavefront per sequence, reduces them.  (A last-workgroup-done fusion of
//     the two stages needs agent-scope release/acquire, which on gfx950 writes
//     back and invalidates the XCD's whole L2 in every workgroup: measured at
//     +35-55 us per sweep, against 1-3 us for the second launch.)
//
// Memory pattern: lane l of a wave reads 16 contiguous bytes at column
// c*CW + l*EPL of its row (CW = 64 lanes x EPL elements), so each load
// instruction of a wave fetches 1 KiB of one row; RPI rows x U chunks are in
// flight per wave, with the non-temporal hint (each weight byte is read once
// per sweep).  Rows are dealt to the waves of the whole grid round-robin, so
// at any moment the grid streams one contiguous window of the matrix.  The
// first group of loads is issued before the prologue so HBM is busy while the
// norms are computed.  Grids are a multiple of the CU count so every CU gets
// the same number of workgroups.
//
// Sums are FP32 in a fixed order (per lane over its chunks, then DPP moves
// within each 16-lane row and the four row sums in row order), so results do
// not depend on grid size or timing; the argmax order (value, then lower
// index) is associative, so neither does the draft.
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"

namespace mtp {

// Dot of 8 BF16 weights with 8 BF16 activations, accumulated in order.
__device__ __forceinline__ float dot8_bf16(const uint4 &w, const uint4 &a, float acc)
{
    acc = fmaf(bf16_lo(w.x), bf16_lo(a.x), acc);
    acc = fmaf(bf16_hi(w.x), bf16_hi(a.x), acc);
    acc = fmaf(bf16_lo(w.y), bf16_lo(a.y), acc);
    acc = fmaf(bf16_hi(w.y), bf16_hi(a.y), acc);
    acc = fmaf(bf16_lo(w.z), bf16_lo(a.z), acc);
    acc = fmaf(bf16_hi(w.z), bf16_hi(a.z), acc);
    acc = fmaf(bf16_lo(w.w), bf16_lo(a.w), acc);
    acc = fmaf(bf16_hi(w.w), bf16_hi(a.w), acc);
    return acc;
}

// Dot of 4 E4M3FN codes (one dword) with 4 BF16 activations (two dwords).
// gfx950's v_cvt_pk_f32_fp8 decodes OCP E4M3FN exactly.
__device__ __forceinline__ float dot4_fp8(uint32_t q, uint32_t a01, uint32_t a23, float acc)
{
    typedef float f2 __attribute__((ext_vector_type(2)));
    const f2 d01 = __builtin_amdgcn_cvt_pk_f32_fp8(int(q), false);
    const f2 d23 = __builtin_amdgcn_cvt_pk_f32_fp8(int(q), true);
    acc = fmaf(d01.x, bf16_lo(a01), acc);
    acc = fmaf(d01.y, bf16_hi(a01), acc);
    acc = fmaf(d23.x, bf16_lo(a23), acc);
    acc = fmaf(d23.y, bf16_hi(a23), acc);
    return acc;
}

// Sum of a value over the 64 lanes of a wave, the same in every lane: DPP
// moves within each 16-lane row (pairs, quads, half-row mirror, row mirror),
// then the four row sums read into scalars and added in row order.  No LDS
// round trips (an xor butterfly of lane shuffles costs six).
__device__ __forceinline__ float row_sum64(float v)
{
    auto dpp = [](float x, auto ctrl) {
        return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), decltype(ctrl)::value,
                                                       0xF, 0xF, true));
    };
    v += dpp(v, std::integral_constant<int, 0xB1>{});   // quad_perm [1, 0, 3, 2]
    v += dpp(v, std::integral_constant<int, 0x4E>{});   // quad_perm [2, 3, 0, 1]
    v += dpp(v, std::integral_constant<int, 0x141>{});  // row_half_mirror
    v += dpp(v, std::integral_constant<int, 0x140>{});  // row_mirror
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
    return ((r0 + r1) + r2) + r3;
}

// Weight stream loads.  With NT the load carries the non-temporal hint: the
// weights are read once per sweep, so they should not displace the cached
// activations and workspace.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
template <bool NT>
__device__ __forceinline__ uint4 ld_weights(const char *p)
{
    if (NT) {
        const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
        return make_uint4(v.x, v.y, v.z, v.w);
    }
    return *reinterpret_cast<const uint4 *>(p);
}

template <bool FP8, int PRO, int EPI, int RPI, int U, bool NT = true, int BS = 256, bool DB = false>
__global__ __launch_bounds__(BS) void row_gemv_kernel(RowGemvArgs a)
{
    extern __shared__ uint4 lds_raw[];
    __shared__ float red[32];
    __shared__ float best_v_s[16];
    __shared__ uint32_t best_i_s[16];
    uint16_t *act = reinterpret_cast<uint16_t *>(lds_raw);

    const int b = blockIdx.y;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    // the wave index is uniform across the wave; saying so keeps the row
    // numbers, and the buffer resources built from them, in scalar registers
    const int wid = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int K = a.K;

    constexpr int EPL = FP8 ? 16 : 8;  // elements per 16-byte load
    constexpr int CW = kWave * EPL;    // columns per wave-wide load
    constexpr int ESZ = FP8 ? 1 : 2;   // bytes per weight element
    const int nchunks = (K + CW - 1) / CW;
    const int wpb = BS / kWave;
    const int Wt = gridDim.x * wpb;
    const int gw = blockIdx.x * wpb + wid;
    const int N = a.N;
    const char *Wb = reinterpret_cast<const char *>(a.W);

    // Row ownership: interleaved (row r goes to wave r mod Wt) or, with
    // a.contig_rows > 0, contiguous blocks of that many rows per wave.
    int r_begin = gw, r_end = N, r_inner = Wt;
    if (a.contig_rows > 0) {
        r_begin = gw * a.contig_rows;
        r_end = min(N, r_begin + a.contig_rows);
        r_inner = 1;
    }
    const int r_outer = r_inner * RPI;

    uint4 wv[RPI][U];
    // The front (eh_proj: a few rows per wave) issues every load (a row past
    // r_end reads row 0, a column past K column 0, values that are never
    // used): no branches and nothing computed from the loaded values at load
    // time, so the compiler counts the loads exactly and waits for a group
    // only where it is multiplied.  The head sweeps (tens of
    // rows per wave) branch around such loads; measured, the branch-free form
    // costs them about 5% of bandwidth.
    auto load_into = [&](uint4(&dst)[RPI][U], int r0, int c0) {
#pragma unroll
        for (int k = 0; k < RPI; ++k) {
            const int r = r0 + k * r_inner;
            const bool rok = r < r_end;
            if constexpr (PRO == PRO_FRONT) {
                // the values read in place of a row past r_end or a column past
                // K are never used: columns past K are skipped by the
                // multiply-add and rows past r_end are not stored
                const char *row = Wb + size_t(rok ? r : 0) * size_t(K) * ESZ;  // row 0 exists
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int col = (c0 + u) * CW + lane * EPL;
                    dst[k][u] = ld_weights<NT>(row + size_t(col < K ? col : 0) * ESZ);
                }
            } else {
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int col = (c0 + u) * CW + lane * EPL;
                    dst[k][u] = make_uint4(0, 0, 0, 0);
                    if (rok && col < K)
                        dst[k][u] = ld_weights<NT>(Wb + (size_t(r) * size_t(K) + size_t(col)) * ESZ);
                }
            }
        }
    };
    auto load_group = [&](int r0, int c0) { load_into(wv, r0, c0); };
    // The single-sequence head's last three passes on demand (row_ctr set):
    // the waves do not stream equally fast (its loops ended up to 9 us apart
    // with fixed shares).  Pool p is the waves of workgroups w with
    // (w / 8) mod npool = p, one workgroup per XCD at 512 workgroups.  A take
    // is an atomic every lane issues, lane 0's inside the counters' range,
    // the others touching no memory.
    // One row per pass only (RPI is a template argument, so the FP8 head, two
    // rows per pass, holds no tail code): compiled into the FP8 head the tail
    // made it 8 us slower (139 -> 147 us) even in calls that never take it.
    const bool dyn = EPI == EPI_ARGMAX && RPI == 1 && a.row_ctr && gridDim.y == 1 &&
                     a.contig_rows == 0 && nchunks <= U && N / r_outer >= 5;
    const int PS = dyn ? N / r_outer - 3 : 0x7FFFFFFF, RS = dyn ? PS * r_outer : 0;
    const int npool = max(1, min(kRowPools, int(gridDim.x) / 8));
    const int pool = (int(blockIdx.x) / 8) % npool;
    const __amdgpu_buffer_rsrc_t ctr_rs = __builtin_amdgcn_make_buffer_rsrc(
        a.row_ctr, 0, dyn ? kRowPools * kCtrStride : 0, 0x00020000);
    auto take = [&]() {
        return uint32_t(__builtin_amdgcn_raw_ptr_buffer_atomic_add_i32(
            1, ctr_rs, lane == 0 ? pool * kCtrStride : int(0x80000000u), 0, 0));
    };
    uint32_t gt0 = 0, gt1 = 0;
    // ---- prologue: the BF16 activation vector act[0..K) in LDS -------------
    // The first weight group does not depend on the activation, so its loads
    // are issued before the norm completes.  In the front the norm's loads go
    // first: completion is counted in issue order, so the norm can finish
    // while the weights are still arriving.
    if constexpr (PRO == PRO_FRONT) {
        // the counters of the head launched next start at zero
        if (a.zero_ctr && blockIdx.x == 0 && b == 0 && tid < kRowPools)
            a.zero_ctr[tid * (kCtrStride / 4)] = 0u;
        // K = 2H: [enorm(embed[token]) | hnorm(hidden[b])]
        const int H = K / 2;
        const uint32_t tok = a.tokens[b];
        const bool tok_ok = tok < uint32_t(a.vocab);
        const uint16_t *erow = a.embed + (tok_ok ? size_t(tok) * size_t(H) : 0);
        const DualNormIn nv =
            dual_norm_load(erow, tok_ok, a.enorm_w, a.hidden + size_t(b) * H, a.hnorm_w, H);
        load_group(r_begin, 0);
        __builtin_amdgcn_sched_barrier(0);  // keep the weight loads ahead of the norm
        dual_norm_store(nv, H, a.eps, act, act + H, red);
    } else {
        // K = H: shared_head.norm(x[b]), the first weight group in flight (the
        // tail's first two counts before it: they come back under the norm)
        if (dyn) {
            gt0 = take();
            gt1 = take();
        }
        load_group(r_begin, 0);
        single_norm(a.xin + size_t(b) * K, a.norm_w, K, a.eps, act, red);
    }
    __syncthreads();

    // ---- row sweep ---------------------------------------------------------
    float best_v = -INFINITY;
    uint32_t best_i = 0xFFFFFFFFu;
    float acc[RPI];
#pragma unroll
    for (int k = 0; k < RPI; ++k)
        acc[k] = 0.f;

    // multiply-add one group of weights into acc
    auto mac_group = [&](const uint4(&w)[RPI][U], int c0) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int col = (c0 + u) * CW + lane * EPL;
            if (col < K) {
                if (!FP8) {
                    const uint4 av = *reinterpret_cast<const uint4 *>(act + col);
#pragma unroll
                    for (int k = 0; k < RPI; ++k)
                        acc[k] = dot8_bf16(w[k][u], av, acc[k]);
                } else {
                    const uint4 a0 = *reinterpret_cast<const uint4 *>(act + col);
                    const uint4 a1 = *reinterpret_cast<const uint4 *>(act + col + 8);
#pragma unroll
                    for (int k = 0; k < RPI; ++k) {
                        float s = acc[k];
                        s = dot4_fp8(w[k][u].x, a0.x, a0.y, s);
                        s = dot4_fp8(w[k][u].y, a0.z, a0.w, s);
                        s = dot4_fp8(w[k][u].z, a1.x, a1.y, s);
                        s = dot4_fp8(w[k][u].w, a1.z, a1.w, s);
                        acc[k] = s;
                    }
                }
            }
        }
    };
    // Logits of the wave's finished rows (row, value), written kStage at a
    // time by the whole wave: lane l writes entries l and l + 64.
    constexpr int kStage = 128;
    __shared__ uint32_t st_r[BS / kWave][kStage];
    __shared__ uint16_t st_v[BS / kWave][kStage];
    int nst = 0;  // the same in every lane of the wave
    auto flush_logits = [&]() {
        if (lane < nst)
            a.logits[size_t(b) * N + st_r[wid][lane]] = st_v[wid][lane];
        if (lane + kWave < nst)
            a.logits[size_t(b) * N + st_r[wid][lane + kWave]] = st_v[wid][lane + kWave];
        nst = 0;
    };
    // the finished rows r0 + k r_inner: round, store, argmax bookkeeping
    auto finish_rows = [&](int r0) {
#pragma unroll
        for (int k = 0; k < RPI; ++k) {
            const int r = r0 + k * r_inner;
            const float sum = row_sum64(acc[k]);
            acc[k] = 0.f;
            if (r < r_end) {
                if (EPI == EPI_STORE) {
                    if (lane == 0)
                        a.out[size_t(b) * N + r] = uint16_t(f32_to_bf16_bits(sum));
                } else {
                    const float z = FP8 ? sum * a.scale[r] : sum;
                    const uint32_t lb = f32_to_bf16_bits(z);
                    // Lane 0 stores every rounded logit into the workspace's
                    // small sink (its lines stay in L2), with or without a
                    // logits buffer: without a store per row the head streams
                    // its rows about 5% slower (B = 1 BF16 head call 278
                    // against 263 us).  The logits themselves are staged per
                    // wave and written 128 at a time: stored to the buffer
                    // row by row they cost 1.5 us per head call (BF16 265.1
                    // against 263.5 us, FP8 139.0 against 137.5).
                    if (lane == 0) {
                        *(reinterpret_cast<uint16_t *>(a.partials + size_t(b) * kMaxHeadBlocks +
                                                       kLogitSinkFirst) +
                          (r & (kLogitSinkSlots - 1))) = uint16_t(lb);
                        if (a.logits) {
                            st_r[wid][nst] = uint32_t(r);
                            st_v[wid][nst] = uint16_t(lb);
                        }
                    }
                    if (a.logits && ++nst == kStage)
                        flush_logits();
                    const float lv = __uint_as_float(lb << 16);
                    if (better(lv, uint32_t(r), best_v, best_i)) {
                        best_v = lv;
                        best_i = uint32_t(r);
                    }
                }
            }
        }
    };

    if constexpr (DB) {
        // Double-buffered: the wave's groups in order (row pass, then column
        // group), the next one's loads issued before the current one is
        // multiplied, so a wave always has a group in flight.  Loads past the
        // wave's last group read row 0 (valid, cached) and are never used.
        const int gpr = (nchunks + U - 1) / U;  // groups per row pass
        const int passes = r_begin < r_end ? (r_end - r_begin + r_outer - 1) / r_outer : 0;
        const int G = passes * gpr;
        uint4 wb[RPI][U];
        auto at = [&](int q, int &r0, int &c0) {
            const int p = q / gpr;
            r0 = r_begin + p * r_outer;
            c0 = (q - p * gpr) * U;
        };
        auto consume = [&](const uint4(&w)[RPI][U], int q) {
            int r0, c0;
            at(q, r0, c0);
            mac_group(w, c0);
            if (c0 + U >= nchunks)
                finish_rows(r0);
        };
        for (int q = 0; q < G; q += 2) {
            int r1, c1, r2, c2;
            at(q + 1, r1, c1);
            load_into(wb, r1, c1);
            consume(wv, q);
            at(q + 2, r2, c2);
            load_into(wv, r2, c2);
            if (q + 1 < G)
                consume(wb, q + 1);
        }
    } else {
        // Every pass but the last three deals rows round-robin; with row_ctr
        // (one sequence, the eh_proj launch before this one having cleared the
        // counters) the rows from RS on go in units of RPI consecutive rows
        // from the wave's pool instead (the tail below).
        bool have_group = true;
        int pass = 0;
        for (int r0 = r_begin; r0 < r_end && pass < PS; r0 += r_outer, ++pass) {
            for (int c0 = 0; c0 < nchunks; c0 += U) {
                if (!have_group)
                    load_group(r0, c0);
                have_group = false;
                mac_group(wv, c0);
            }
            finish_rows(r0);
        }
        if (dyn) {
            // Tail: unit g of the wave's pool p is rows RS + (p + npool g) RPI ..;
            // the wave takes its next unit when it starts one, so a count is
            // two units ahead of its use (the first two were taken in the
            // prologue), and the wait for a unit's loads already covers the
            // count taken before them.  Counts increase: the first unit past
            // the last row ends the loop.
            r_inner = 1;
            auto unit_row = [&](uint32_t g) {
                return RS + (pool + npool * int(__builtin_amdgcn_readfirstlane(g))) * RPI;
            };
            int r0 = unit_row(gt0);
#pragma unroll 1
            while (r0 < N) {
                load_group(r0, 0);
                gt0 = take();
                mac_group(wv, 0);
                finish_rows(r0);
                r0 = unit_row(gt1);
                if (r0 >= N)
                    break;
                load_group(r0, 0);
                gt1 = take();
                mac_group(wv, 0);
                finish_rows(r0);
                r0 = unit_row(gt0);
            }
        }
    }

    if (EPI == EPI_ARGMAX && a.logits)
        flush_logits();
    if (EPI == EPI_ARGMAX) {
        // every lane holds the same best (the sums were all-reduced)
        if (lane == 0) {
            best_v_s[wid] = best_v;
            best_i_s[wid] = best_i;
        }
        __syncthreads();
        if (tid == 0) {
            float bv = best_v_s[0];
            uint32_t bi = best_i_s[0];
            for (int w = 1; w < wpb; ++w)
                if (better(best_v_s[w], best_i_s[w], bv, bi)) {
                    bv = best_v_s[w];
                    bi = best_i_s[w];
                }
            a.partials[size_t(b) * kMaxHeadBlocks + blockIdx.x] = Partial{bv, bi};
        }
    }
}

// Second argmax stage: one wavefront per sequence reduces its partials and
// writes the draft (MTP_DRAFT_INVALID when the sequence's token is out of
// range).  One wave needs no LDS and no barrier: eight partials per lane are
// loaded before any is compared (one memory latency per 512 partials, which
// covers the heads' grids), each 16-lane row is reduced with DPP moves, and
// the four row winners are compared in row order from v_readlane.  The
// (value, lower index) order is total, so any reduction tree picks the same
// winner.  (A 256-thread workgroup with LDS-permute butterflies took 4.5 us
// per call.)
__global__ __launch_bounds__(64) void argmax_final_kernel(const Partial *__restrict__ partials,
                                                          int nparts, const uint32_t *tokens,
                                                          int vocab, uint32_t *draft)
{
    const int b = blockIdx.x;
    const int lane = threadIdx.x;
    // the token check's load (every lane reads the same word) goes out
    // together with the partials' loads and is used only at the end
    const uint32_t tk = tokens ? tokens[b] : 0u;
    float bv = -INFINITY;
    uint32_t bi = 0xFFFFFFFFu;
    // a slot past nparts re-reads the last partial and is skipped
    constexpr int PER = 8;
    for (int p0 = lane; p0 < nparts; p0 += PER * kWave) {
        Partial q[PER];
#pragma unroll
        for (int u = 0; u < PER; ++u)
            q[u] = partials[size_t(b) * kMaxHeadBlocks + min(p0 + u * kWave, nparts - 1)];
#pragma unroll
        for (int u = 0; u < PER; ++u)
            if (p0 + u * kWave < nparts && better(q[u].val, q[u].idx, bv, bi)) {
                bv = q[u].val;
                bi = q[u].idx;
            }
    }
    auto step = [&](auto ctrl) {
        constexpr int C = decltype(ctrl)::value;
        const float ov = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(bv), C, 0xF, 0xF, false));
        const uint32_t oi = uint32_t(__builtin_amdgcn_mov_dpp(int(bi), C, 0xF, 0xF, false));
        if (better(ov, oi, bv, bi)) {
            bv = ov;
            bi = oi;
        }
    };
    step(std::integral_constant<int, 0xB1>{});   // quad_perm [1, 0, 3, 2]
    step(std::integral_constant<int, 0x4E>{});   // quad_perm [2, 3, 0, 1]
    step(std::integral_constant<int, 0x141>{});  // row_half_mirror
    step(std::integral_constant<int, 0x140>{});  // row_mirror
    float rv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(bv), 0));
    uint32_t ri = uint32_t(__builtin_amdgcn_readlane(int(bi), 0));
#pragma unroll
    for (int r = 1; r < 4; ++r) {
        const float v = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(bv), 16 * r));
        const uint32_t i = uint32_t(__builtin_amdgcn_readlane(int(bi), 16 * r));
        if (better(v, i, rv, ri)) {
            rv = v;
            ri = i;
        }
    }
    if (lane == 0) {
        if (tokens && tk >= uint32_t(vocab))
            ri = 0xFFFFFFFFu;
        draft[b] = ri;
    }
}

// ---------------------------------------------------------------------------
// Host launchers
// ---------------------------------------------------------------------------

template <bool FP8, int PRO, int EPI, int RPI, int U, bool DB = false>
static hipError_t launch_one(const RowGemvArgs &a, int grid, int batch, hipStream_t s,
                             int *grid_out)
{
    if (grid_out)
        *grid_out = grid;
    const size_t lds = align256(size_t(a.K) * 2);
    hipLaunchKernelGGL((row_gemv_kernel<FP8, PRO, EPI, RPI, U, true, 256, DB>), dim3(grid, batch),
                       dim3(256), lds, s, a);
    return hipGetLastError();
}

int device_cu_count()
{
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess)
        return 256;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
        return 256;
    return n;
}

// Workgroups: `per_cu` per CU (so every CU carries the same load), but no
// more than the rows need (4 waves x rpi rows per workgroup pass).
static int grid_for(int N, int rpi, int per_cu, int cu_count)
{
    int grid = cu_count * per_cu;
    const int need = (N + 4 * rpi - 1) / (4 * rpi);
    if (grid > need)
        grid = need;
    if (grid > kLogitSinkFirst)  // the partial slots above hold the no-logits sink
        grid = kLogitSinkFirst;
    return grid < 1 ? 1 : grid;
}

// BF16 weights: 512 columns per wave-wide load.  U = chunks per row held in
// flight (the whole row when it fits), RPI = rows per wave pass.
template <int PRO, int EPI>
static hipError_t launch_bf16(const RowGemvArgs &a, int per_cu, int batch, hipStream_t s, int cus,
                              int *grid_out)
{
    const int nch = (a.K + 511) / 512;
#define MTP_BF16(RPI, U) \
    return launch_one<false, PRO, EPI, RPI, U>(a, grid_for(a.N, RPI, per_cu, cus), batch, s, \
                                               grid_out)
    if (nch <= 1) MTP_BF16(4, 1);
    if (nch <= 2) MTP_BF16(4, 2);
    if (nch <= 4) MTP_BF16(2, 4);
    if (nch <= 8) MTP_BF16(2, 8);
    if (nch <= 12) MTP_BF16(1, 12);
    if (nch <= 16) MTP_BF16(1, 16);
    if (nch <= 24) MTP_BF16(1, 24);
    MTP_BF16(1, 16);
#undef MTP_BF16
}

// FP8 codes: 1024 columns per wave-wide load.
static hipError_t launch_fp8_head(const RowGemvArgs &a, int per_cu, int batch, hipStream_t s,
                                  int cus, int *grid_out)
{
    const int nch = (a.K + 1023) / 1024;
#define MTP_FP8(RPI, U)                                                                         \
    return launch_one<true, PRO_HEADNORM, EPI_ARGMAX, RPI, U>(a, grid_for(a.N, RPI, per_cu, cus), \
                                                               batch, s, grid_out)
    if (nch <= 1) MTP_FP8(4, 1);
    if (nch <= 2) MTP_FP8(4, 2);
    if (nch <= 4) MTP_FP8(2, 4);
    if (nch <= 6) MTP_FP8(2, 6);
    MTP_FP8(2, 8);
#undef MTP_FP8
}

// eh_proj: a few rows per wave, so the groups are double-buffered (half a
// row each at K = 2H = 12288) to keep every wave streaming; short rows take
// the single-buffered sweep.
hipError_t launch_eh_proj(const RowGemvArgs &a, int batch, hipStream_t s)
{
    const int nch = (a.K + 511) / 512;
    if (nch <= 8)
        return launch_bf16<PRO_FRONT, EPI_STORE>(a, 2, batch, s, device_cu_count(), nullptr);
    return launch_one<false, PRO_FRONT, EPI_STORE, 1, 12, true>(
        a, grid_for(a.N, 1, 2, device_cu_count()), batch, s, nullptr);
}

hipError_t launch_head(const RowGemvArgs &a, bool fp8, int batch, hipStream_t s)
{
    const int cus = device_cu_count();
    int grid = 0;
    // two 4-wave workgroups per CU for both heads: measured on the FP8 codes,
    // 2 per CU streams ~5% faster than 3, 4 or 5 (and than 1)
    const hipError_t e = fp8 ? launch_fp8_head(a, 2, batch, s, cus, &grid)
                             : launch_bf16<PRO_HEADNORM, EPI_ARGMAX>(a, 2, batch, s, cus, &grid);
    if (e != hipSuccess)
        return e;
    return launch_argmax_final(a.partials, grid, a.tokens, a.vocab, a.draft, batch, s);
}

hipError_t launch_argmax_final(const Partial *partials, int nparts, const uint32_t *tokens,
                               int vocab, uint32_t *draft, int batch, hipStream_t s)
{
    hipLaunchKernelGGL(argmax_final_kernel, dim3(batch), dim3(kWave), 0, s, partials, nparts,
                       tokens, vocab, draft);
    return hipGetLastError();
}

}  // namespace mtp
