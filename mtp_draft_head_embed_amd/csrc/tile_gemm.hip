// tile_gemm.hip -- the batched sweep's two weight streams for 2 <= B <= 16
// sequences on matrix cores, one 16-row weight tile per workgroup at a time:
//   * lm_head (`dense_gemv` / `dense_gemv_fp8w` of metrale_model_arch/
//     glm5next_mtp_head.rs, `forward_one`, run for B sequences at once) with
//     the per-workgroup argmax partials as its epilogue (H <= 6144);
//   * eh_proj over [enorm(embed[token]) | hnorm(hidden)] (the same page's
//     `forward_one`: the embedding row read by pointer, the two vanilla norms,
//     the concat and the projection), K split four ways, the two norms computed
//     in the prologue, FP32 partial sums out (H a multiple of 1024 up to 6144).
//
// Work split.  16-row tiles of the weight matrix are dealt round-robin to the
// workgroups (one 8-wave workgroup per CU; the head's last three to four
// rounds on demand instead, from counters in the workspace), and the 8 waves
// split each tile's K (or the workgroup's K split) into 8 equal slices.  A workgroup therefore
// reads 16 whole rows (or row quarters) at a time, and the grid a window of
// 256 such blocks: a streaming probe reads 12 KiB rows 8% faster this way than
// with one tile per wave (7.15 against 6.63 TB/s), 6 KiB rows about 1% faster.
//
// Per wave:
//   * its slice of the B activation rows stays in registers for the whole
//     call, as MFMA A fragments (at most 24 x 16 bytes per lane), so nothing is
//     staged in LDS and B = 16 needs no K chunks;
//   * the weight slice comes in chunks of 2 NSEG 16-byte loads per lane (NSEG
//     128-byte segments of each of the 16 rows; every load instruction reads
//     whole 128-byte lines of 8 rows), double-buffered: the next chunk's loads
//     are in flight while this one is multiplied;
//   * each chunk is re-laid through the wave's 2 KiB LDS scratch into MFMA
//     layout (piece p of row r at slot p ^ ((r >> 1) & 7), conflict-free) and
//     multiplied with v_mfma_f32_16x16x32_bf16, FP8 codes decoded to BF16 in
//     registers (exact); the FP8 row scale multiplies the FP32 sum once.
// The 8 slice sums of a tile meet in LDS and are added in wave order; waves
// 0-3 finish the tile's 16 x 16 outputs (rounded logits and a running (max,
// lowest index) per (sequence, tile row), or FP32 partial sums) into an LDS
// buffer that goes to memory after the loop.  The barrier that publishes the
// slice sums waits only for LDS, so the prefetched chunks stay in flight
// across it.
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"
#include "mfma_util.hpp"

namespace mtp {

namespace {

enum { TILE_HEAD = 0, TILE_FRONT = 1 };
constexpr int kFrontSplits = 4;  // K splits of the front: each inside one half

struct TileArgs {
    const void *W;        // [N][K] BF16, or E4M3FN codes (FP8 head)
    const float *scale;   // [N] per-row scale (FP8 head)
    int N, K, B;
    // head
    const uint16_t *A;    // [B][K] BF16 normed activations
    uint16_t *logits;     // [B][N] BF16 or null
    Partial *partials;    // [B][kMaxHeadBlocks]
    uint32_t *tile_ctr;   // kTilePools counters kCtrStride bytes apart, zero at launch
    // front (K = 2H, N = H)
    const uint16_t *embed;
    int vocab;
    const uint32_t *tokens;
    const uint16_t *hidden;
    const uint16_t *enorm_w, *hnorm_w;
    float eps;
    float *out_f32;       // [kFrontSplits][B][H] partial sums
};

}  // namespace

// NSEG: 128-byte segments of each row per chunk; CH: chunks per wave per tile
// (1 or 2).  A wave's slice of a row is CH * NSEG * 128 bytes.
template <int MODE, bool FP8, int NSEG, int CH>
__global__ __launch_bounds__(512) void tile_gemm_kernel(TileArgs a)
{
    static_assert(CH == 1 || CH == 2, "one or two chunks per tile");
    constexpr bool HEAD = MODE == TILE_HEAD;
    static_assert(HEAD || (!FP8 && CH == 1), "the front streams BF16 in one chunk");
    constexpr int NL = 2 * NSEG;          // loads per lane per chunk
    constexpr int SPS = FP8 ? 4 : 2;      // 32-column k-steps per 128-byte segment
    constexpr int NA = CH * NSEG * SPS;   // A fragments per lane
    constexpr int SB = CH * NSEG * 128;   // slice bytes per row per wave
    constexpr int ESZ = FP8 ? 1 : 2;
    // output staging: BF16 logits (head) or FP32 partial sums (front) of up
    // to NBUF tiles, [tile % NBUF][sequence][tile row]
    constexpr int NBUF = HEAD ? 64 : 16;
    using OutT = std::conditional_t<HEAD, uint16_t, float>;
    __shared__ __attribute__((aligned(16))) char xs_all[8 * 2048];
    __shared__ f32x4 red[2][8][kWave];
    __shared__ __attribute__((aligned(16))) OutT ob[NBUF][16][16];
    // front: the split's half of the 16 normed rows, rows padded by 16 bytes
    // so that the 16 lanes of a fragment read hit distinct banks
    constexpr int XLS = NSEG * 512 + 8;
    __shared__ __attribute__((aligned(16))) uint16_t xl[HEAD ? 8 : 16 * XLS];
    // head: the tile of the workgroup's s-th slot at s % 128 (outlives the
    // NBUF slots whose outputs wait in ob)
    __shared__ int slot_tile[HEAD ? 128 : 1];

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wid = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int nl = lane & 15;  // weight row within a tile / batch row of A
    const int g = lane >> 4;   // k-slot group
    const int N = a.N, K = a.K, B = a.B;
    const int rowb = K * ESZ;  // bytes per weight row
    char *xs = xs_all + wid * 2048;
    const char *Wb = reinterpret_cast<const char *>(a.W);
    const int T16 = (N + 15) / 16;
    const int G = int(gridDim.x);

    // Tiles to workgroups.  A tile at or past T16 is empty: its loads read
    // zero without touching memory and it stores nothing.
    //   head: slot s < RS of workgroup w holds tile t0 + s G.  Workgroups are
    //   dispatched to the 8 XCDs in turn, each XCD with its own L2, and are
    //   numbered here XCD by XCD, so neighbouring tiles meet in one L2
    //   (measured while the logits were stored tile by tile: numbered in
    //   dispatch order, they cost the B = 16 head another 15 us (FP8) and
    //   22 us (BF16) at V = 154 880).  The last three to four rounds of tiles,
    //   from RS G on, are dealt on demand instead: the XCDs do not stream
    //   equally fast (at V = 154 880, B = 16 FP8: 3.11 us per tile on half of
    //   them, 3.35 on the other half), and with fixed shares the slower half
    //   finished 8 us after the faster.  They form P pools, pool p holding
    //   tiles RS G + p + P i, shared by the workgroups w with (w / 8) mod P = p
    //   (four per XCD at G = 256); a workgroup's next tile in its pool is the
    //   count its pool's counter held when it added one.  One counter for all
    //   tiles, taken about 75 times per us, did not keep up (the B = 16 FP8
    //   sweep took 213 us against 181); P counters on their own 4 KiB pages,
    //   taken only in the tail, do.
    //   front: workgroup w takes K split w % 4 of tiles w / 4 + i G / 4, so its
    //   A fragments (one split) serve all its tiles.
    int t0, tstride, split = 0;
    if constexpr (HEAD) {
        t0 = (G % 8 == 0) ? (int(blockIdx.x) % 8) * (G / 8) + int(blockIdx.x) / 8
                          : int(blockIdx.x);
        tstride = G;
    } else {
        split = int(blockIdx.x) % kFrontSplits;
        t0 = int(blockIdx.x) / kFrontSplits;
        tstride = G / kFrontSplits;
    }
    // front: the workgroup's tix-th tile (>= 1 tile: the grid has no idle workgroup)
    const int ntile = (T16 - 1 - t0) / tstride + 1;
    auto tile_of = [&](int tix) {
        if constexpr (HEAD)
            return __builtin_amdgcn_readfirstlane(slot_tile[tix & 127]);
        else
            return t0 + tix * tstride;
    };
    // head: static slots, pools, this workgroup's pool
    const int RS = max(2, T16 / G - 3);
    const int npool = max(1, min(kTilePools, G / 8));
    const int pool = (int(blockIdx.x) / 8) % npool;
    const __amdgpu_buffer_rsrc_t ctr_rs = __builtin_amdgcn_make_buffer_rsrc(
        HEAD ? a.tile_ctr : nullptr, 0, HEAD ? kTilePools * kCtrStride : 0, kBufFlags);
    // Slot s's tile, for s >= 2.  Every lane issues the atomic (no branch, so
    // the loads around it are counted exactly); only thread 0's, and only for
    // a pooled slot, lies inside the counters' range, every other one outside
    // it, which touches no memory.  Thread 0 gets the count back; publish()
    // turns it into the tile.
    auto take = [&](int s) {
        const bool real = tid == 0 && s >= RS;
        return uint32_t(__builtin_amdgcn_raw_ptr_buffer_atomic_add_i32(
            1, ctr_rs, real ? pool * kCtrStride : int(0x80000000u), 0, 0));
    };
    auto publish = [&](int s, uint32_t g) {  // thread 0: slot s's tile into slot_tile
        if (tid == 0)
            slot_tile[s & 127] = s < RS ? t0 + s * G : RS * G + pool + npool * int(g);
    };
    // the wave's slice of each row (bytes): head, wave w of the whole row;
    // front, wave w of the split's H / 2 columns (H = 1024 NSEG: SB bytes)
    const int sb0 = HEAD ? wid * SB : (split * (K / kFrontSplits)) * 2 + wid * SB;

    // Chunk c of a tile: load u reads rows 0-7 (u even) or 8-15 (u odd) of
    // segment u / 2, 16 bytes per lane.  Rows past N lie outside the resource
    // and columns past K are sent outside it: both read zero.  An empty tile
    // (rows from N on) gets an empty range, so its loads read zero without
    // touching memory; the loops below issue them unconditionally.
    auto load_chunk = [&](uint4 (&raw)[NL], int tile, int c) {
        const int r0 = min(N, tile * 16);
        const int r1 = min(N, r0 + 16);
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<char *>(Wb) + size_t(r0) * size_t(rowb), 0, (r1 - r0) * rowb, kBufFlags);
        const int seg0 = sb0 + c * NSEG * 128 + (lane & 7) * 16;
        const int vo0 = (lane >> 3) * rowb + seg0;
#pragma unroll
        for (int u = 0; u < NL; ++u) {
            const int colb = seg0 + (u >> 1) * 128;
            const int vo = vo0 + ((u & 1) ? 8 * rowb : 0) + (u >> 1) * 128;
            raw[u] = ld_buf16(rs, colb < rowb ? vo : int(0x80000000u));
        }
        // keep the chunk's loads together and in program order: the waits
        // below count on chunks completing one after the other
        __builtin_amdgcn_sched_barrier(0);
    };

    // A fragments: step (s, q) of the slice covers columns
    //   FP8:  slice byte sb0 + 128 s + 64 (q >> 1) + 16 g + 8 (q & 1), 8 columns
    //   BF16: slice byte sb0 + 128 s + 64 q + 16 g, 8 columns
    // -- the columns the re-laid weight pieces hold for (g, step).  Columns
    // past K are zero; batch rows past B take row B - 1 (their outputs are
    // dropped, and an MFMA output row depends only on its own A row).
    auto frag_col = [&](int s, int q) {
        const int byte = sb0 + 128 * s + (FP8 ? 64 * (q >> 1) + 16 * g + 8 * (q & 1) : 64 * q + 16 * g);
        return FP8 ? byte : byte / 2;
    };
    uint4 af[NA];
    uint4 rA[NL], rB[NL];
    const int arow = min(nl, B - 1);
    if constexpr (HEAD) {
        const uint16_t *ap = a.A + size_t(arow) * size_t(K);
#pragma unroll
        for (int s = 0; s < CH * NSEG; ++s)
#pragma unroll
            for (int q = 0; q < SPS; ++q) {
                const int col = frag_col(s, q);
                af[s * SPS + q] =
                    col < K ? *reinterpret_cast<const uint4 *>(ap + col) : make_uint4(0, 0, 0, 0);
            }
    } else {
        // The split lies in one half of [enorm(e) | hnorm(h)]: hf = 0, the
        // embedding row of the sequence's token (zero for a token outside the
        // vocabulary); hf = 1, its hidden row.  Wave w loads the whole rows of
        // sequences w and w + 8 (rows past B repeat row B - 1) for their sums
        // of squares, norms the split's half of them (x * w exact, times 1 / r
        // once per row, as the norms of common.hpp do) into LDS, and after a
        // barrier every wave reads its fragments from there.  Loads complete in
        // issue order: the tokens first (one wait), then the rows and the norm
        // weight, then the first weight chunk; the LDS writes go out before the
        // second chunk.
        const int H = N;
        const int hf = split / 2;
        const uint16_t *nw = hf ? a.hnorm_w : a.enorm_w;
        const int ms[2] = {min(wid, B - 1), min(wid + 8, B - 1)};
        uint32_t tk[2] = {0u, 0u};
        if (!hf) {  // workgroup-uniform; the hidden half needs no token
#pragma unroll
            for (int i = 0; i < 2; ++i)
                tk[i] = a.tokens[ms[i]];
        }
        bool sok[2];
        const uint16_t *srow[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            sok[i] = hf || tk[i] < uint32_t(a.vocab);
            srow[i] = hf ? a.hidden + size_t(ms[i]) * size_t(H)
                         : a.embed + (sok[i] ? size_t(tk[i]) * size_t(H) : size_t(0));
        }
        // 16-byte piece p of a row holds columns (p * 64 + lane) * 8 ..; the
        // split's H / 2 columns of the half are pieces p0 .. p0 + NSEG - 1
        constexpr int PPL = 2 * NSEG;  // H / 512
        const int p0 = (split % 2) * NSEG;
        uint4 sv[2][PPL], wv[NSEG];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int p = 0; p < PPL; ++p)
                sv[i][p] = *reinterpret_cast<const uint4 *>(srow[i] + (p * kWave + lane) * 8);
#pragma unroll
        for (int p = 0; p < NSEG; ++p)
            wv[p] = *reinterpret_cast<const uint4 *>(nw + ((p0 + p) * kWave + lane) * 8);
        load_chunk(rA, tile_of(0), 0);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            float ss = 0.f;
#pragma unroll
            for (int p = 0; p < PPL; ++p) {
                const uint32_t w4[4] = {sv[i][p].x, sv[i][p].y, sv[i][p].z, sv[i][p].w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    ss = fmaf(bf16_lo(w4[e]), bf16_lo(w4[e]), ss);
                    ss = fmaf(bf16_hi(w4[e]), bf16_hi(w4[e]), ss);
                }
            }
            ss = wave_sum(ss);
            const float rr = 1.0f / sqrtf(ss / float(H) + a.eps);  // as the norms of common.hpp
            uint16_t *dst = xl + (wid + 8 * i) * XLS;
#pragma unroll
            for (int p = 0; p < NSEG; ++p) {
                // both indices compile-time and the choice made per component:
                // a runtime index, or a choice between the two elements, would
                // move sv to scratch memory
                const bool odd = split & 1;
                const uint4 hi = sv[i][NSEG + p], lo = sv[i][p];
                const uint4 xv = make_uint4(odd ? hi.x : lo.x, odd ? hi.y : lo.y, odd ? hi.z : lo.z,
                                            odd ? hi.w : lo.w);
                const uint32_t x4[4] = {xv.x, xv.y, xv.z, xv.w};
                const uint32_t w4[4] = {wv[p].x, wv[p].y, wv[p].z, wv[p].w};
                uint32_t o[4];
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    o[e] = sok[i] ? pack_bf16x2((bf16_lo(x4[e]) * bf16_lo(w4[e])) * rr,
                                                (bf16_hi(x4[e]) * bf16_hi(w4[e])) * rr)
                                  : 0u;
                *reinterpret_cast<uint4 *>(dst + (p * kWave + lane) * 8) =
                    make_uint4(o[0], o[1], o[2], o[3]);
            }
        }
        load_chunk(rB, tile_of(1), 0);
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");  // the normed rows
        // fragment (s, q): columns frag_col(s, q) - the split's first column
        const int cbase = split * (K / kFrontSplits);
#pragma unroll
        for (int s = 0; s < NSEG; ++s)
#pragma unroll
            for (int q = 0; q < SPS; ++q)
                af[s * SPS + q] =
                    *reinterpret_cast<const uint4 *>(xl + arow * XLS + (frag_col(s, q) - cbase));
    }

    // Multiply chunk C (compile-time) into acc.
    auto compute = [&](uint4 (&raw)[NL], f32x4 &acc, auto cc) {
        constexpr int C = decltype(cc)::value;
#pragma unroll
        for (int j = 0; j < NSEG; ++j) {
            const int wr0 = lane >> 3, wp = lane & 7;
            *reinterpret_cast<uint4 *>(xs + wr0 * 128 + ((wp ^ ((wr0 >> 1) & 7)) * 16)) = raw[2 * j];
            const int wr1 = 8 + wr0;
            *reinterpret_cast<uint4 *>(xs + wr1 * 128 + ((wp ^ ((wr1 >> 1) & 7)) * 16)) =
                raw[2 * j + 1];
            raw[2 * j] = *reinterpret_cast<const uint4 *>(xs + nl * 128 + ((g ^ ((nl >> 1) & 7)) * 16));
            raw[2 * j + 1] =
                *reinterpret_cast<const uint4 *>(xs + nl * 128 + (((4 + g) ^ ((nl >> 1) & 7)) * 16));
        }
#pragma unroll
        for (int j = 0; j < NSEG; ++j)
#pragma unroll
            for (int q = 0; q < SPS; ++q) {
                bf16x8 wf;
                if constexpr (FP8) {
                    const uint4 &r = raw[2 * j + (q >> 1)];
                    wf = (q & 1) ? fp8x8_to_bf16(r.z, r.w) : fp8x8_to_bf16(r.x, r.y);
                } else {
                    wf = as_bf16x8(raw[2 * j + q]);
                }
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    as_bf16x8(af[(C * NSEG + j) * SPS + q]), wf, acc, 0, 0, 0);
            }
    };

    // Thread t < 256 finishes output element t of the 16 x 16 tile: MFMA lane
    // t / 4, element t % 4, i.e. sequence m = 4 (t / 64) + t % 4 and tile row
    // n = (t / 4) % 16.
    const int m_out = 4 * (tid >> 6) + (tid & 3);
    const int n_out = (tid >> 2) & 15;
    auto load_scale = [&](int tile) {
        float sc = 1.0f;
        if (HEAD && FP8 && wid < 4) {
            const int row = tile * 16 + n_out;
            if (row < N)
                sc = a.scale[row];
        }
        return sc;
    };
    float best_v = -INFINITY;
    uint32_t best_i = 0xFFFFFFFFu;
    // The outputs stay in LDS and go to memory after the loop, or whenever
    // NBUF tiles have gathered: logits stored tile by tile between the weight
    // loads cost the B = 16 head 7-10 us (FP8) and 14 us (BF16) at
    // V = 154 880, whatever their grouping into whole lines, against about
    // 1 us for heads that stored after their last weight load.  All 512
    // threads store 16-byte pieces; logits go element by element where a
    // piece is partial or V is not a multiple of 8 (16-byte alignment).
    auto flush = [&](int f0, int f1) {  // tiles [f0, f1), at most NBUF
        if constexpr (HEAD) {
            if (!a.logits)
                return;
            for (int pc = tid; pc < (f1 - f0) * 32; pc += 512) {
                const int tix = f0 + (pc >> 5), m = (pc >> 1) & 15, h = pc & 1;
                const int r0 = slot_tile[tix & 127] * 16 + 8 * h;
                if (m < B && r0 < N) {
                    const uint16_t *src = &ob[tix % NBUF][m][8 * h];
                    uint16_t *dst = a.logits + size_t(m) * N + r0;
                    if (r0 + 8 <= N && (N & 7) == 0) {
                        *reinterpret_cast<uint4 *>(dst) = *reinterpret_cast<const uint4 *>(src);
                    } else {
                        for (int e = 0; e < 8 && r0 + e < N; ++e)
                            dst[e] = src[e];
                    }
                }
            }
        } else {
            // partial sums, 4 rows per piece (N = H is a multiple of 1024)
            for (int pc = tid; pc < (f1 - f0) * 64; pc += 512) {
                const int tix = f0 + (pc >> 6), m = (pc >> 2) & 15, qd = pc & 3;
                const int r0 = tile_of(tix) * 16 + 4 * qd;
                if (m < B && r0 < N)
                    *reinterpret_cast<float4 *>(a.out_f32 + (size_t(split) * B + m) * N + r0) =
                        *reinterpret_cast<const float4 *>(&ob[tix % NBUF][m][4 * qd]);
            }
        }
    };
    auto finish = [&](f32x4 &acc, int tix, int tile, float sc) {
        const int p = tix & 1;
        red[p][wid][lane] = acc;
        acc = f32x4{0.f, 0.f, 0.f, 0.f};
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        if (tix > 0 && tix % NBUF == 0) {
            // the buffer is full (written before the barrier above); empty it
            // before this tile's outputs reuse its first slot
            flush(tix - NBUF, tix);
            asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        }
        if (wid < 4) {
            const float *rf = reinterpret_cast<const float *>(&red[p][0][0]);
            float z = 0.f;
#pragma unroll
            for (int w = 0; w < 8; ++w)
                z += rf[w * 4 * kWave + tid];
            const uint32_t row = uint32_t(tile * 16 + n_out);
            if (row < uint32_t(N) && m_out < B) {
                if constexpr (HEAD) {
                    const uint32_t lb = f32_to_bf16_bits(FP8 ? z * sc : z);
                    ob[tix % NBUF][m_out][n_out] = uint16_t(lb);
                    const float lv = __uint_as_float(lb << 16);
                    if (better(lv, row, best_v, best_i)) {
                        best_v = lv;
                        best_i = row;
                    }
                } else {
                    ob[tix % NBUF][m_out][n_out] = z;
                }
            }
        }
    };

    // The compiler counts loads in flight per code path and, where paths
    // meet, keeps the smaller count.  So the loop issues each prefetch
    // unconditionally (tiles past the last read zero) and puts the conditional
    // memory operations (scale loads) before it: a stricter count then only
    // waits for those older operations, never for the chunk just prefetched.
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
    int nslot;  // slots run (the last may hold an empty tile)
    if constexpr (!HEAD) {
        // tiles alternate between the two buffers, issued in the prologue; an
        // odd count ends with an empty tile
#pragma unroll 1
        for (int t = 0; t < ntile; t += 2) {
            compute(rA, acc, std::integral_constant<int, 0>{});
            finish(acc, t, tile_of(t), 1.0f);
            load_chunk(rA, tile_of(t + 2), 0);
            compute(rB, acc, std::integral_constant<int, 0>{});
            finish(acc, t + 1, tile_of(t + 1), 1.0f);
            load_chunk(rB, tile_of(t + 3), 0);
        }
        nslot = ntile;
    } else if constexpr (CH == 1) {
        // Slots alternate between the two buffers.  Slot s + 2's tile is taken
        // when slot s - 2 is done, published before slot s's barrier and read
        // after it, when its chunk is issued: a count comes back while two
        // tiles stream.  The slots' tiles increase, so the first empty one
        // ends the loop.  Each take is issued before the chunk it precedes, so
        // the wait for that chunk covers it.
        int tA = t0, tB = t0 + G;
        if (tid == 0) {
            slot_tile[0] = tA;
            slot_tile[1] = tB;
        }
        uint32_t gA = take(2);
        float scA = load_scale(tA);
        load_chunk(rA, tA, 0);
        float scB = load_scale(tB);
        uint32_t gB = take(3);
        load_chunk(rB, tB, 0);
        int t = 0;
#pragma unroll 1
        for (; tA < T16; t += 2) {
            compute(rA, acc, std::integral_constant<int, 0>{});
            publish(t + 2, gA);
            finish(acc, t, tA, scA);
            tA = tile_of(t + 2);
            scA = load_scale(tA);
            gA = take(t + 4);
            load_chunk(rA, tA, 0);
            compute(rB, acc, std::integral_constant<int, 0>{});
            publish(t + 3, gB);
            finish(acc, t + 1, tB, scB);
            tB = tile_of(t + 3);
            scB = load_scale(tB);
            gB = take(t + 5);
            load_chunk(rB, tB, 0);
        }
        nslot = t;
    } else {
        // Chunk 0 of every slot in rA, chunk 1 in rB.  Slot s + 2's tile is
        // taken when slot s - 1 is done, published before slot s's barrier and
        // read after it, a slot before its chunks are issued.
        int tc = t0, tn = t0 + G;  // this slot's tile, the next one's
        if (tid == 0) {
            slot_tile[0] = tc;
            slot_tile[1] = tn;
        }
        // the take between the two chunks, where each step issues it (the
        // compiler keeps the smaller count where the paths into the loop meet)
        float sc = load_scale(tc);
        load_chunk(rA, tc, 0);
        uint32_t g = take(2);
        load_chunk(rB, tc, 1);
        int t = 0;
#pragma unroll 1
        for (; tc < T16; ++t) {
            compute(rA, acc, std::integral_constant<int, 0>{});
            load_chunk(rA, tn, 0);
            compute(rB, acc, std::integral_constant<int, 1>{});
            publish(t + 2, g);
            finish(acc, t, tc, sc);
            sc = load_scale(tn);
            g = take(t + 3);
            load_chunk(rB, tn, 1);
            tc = tn;
            tn = tile_of(t + 2);
        }
        nslot = t;
    }

    // the outputs still in LDS
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    flush((nslot - 1) / NBUF * NBUF, nslot);

    if constexpr (HEAD) {
        // Per sequence, the best of the workgroup: the 16 threads of sequence
        // m are lanes 4 n + m % 4 of wave m / 4.
        if (wid < 4) {
#pragma unroll
            for (int msk = 4; msk < kWave; msk <<= 1) {
                const float ov = __shfl_xor(best_v, msk, kWave);
                const uint32_t oi = uint32_t(__shfl_xor(int(best_i), msk, kWave));
                if (better(ov, oi, best_v, best_i)) {
                    best_v = ov;
                    best_i = oi;
                }
            }
            if (n_out == 0 && m_out < B)
                a.partials[size_t(m_out) * kMaxHeadBlocks + blockIdx.x] = Partial{best_v, best_i};
        }
    }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------

template <int MODE, bool FP8, int NSEG, int CH>
static hipError_t launch_tile(const TileArgs &a, int grid, hipStream_t s)
{
    hipLaunchKernelGGL((tile_gemm_kernel<MODE, FP8, NSEG, CH>), dim3(grid), dim3(512), 0, s, a);
    return hipGetLastError();
}

// Whether the tile kernel serves this head: 2 <= B <= 16 and a slice of at
// most 12 segments per wave (H <= 6144 for either dtype).
bool head_tile_fits(int B, int K, bool fp8)
{
    const int seg = (K * (fp8 ? 1 : 2) + 1023) / 1024;
    return B >= 2 && B <= 16 && seg <= (fp8 ? 6 : 12);
}

// One workgroup per CU (or per tile, when the tiles are fewer).  The slice
// per wave is rounded up to 2, 4 or 6 segments per chunk; segments past the
// row read zero.
hipError_t launch_head_tile(const MfmaArgs &m, bool fp8, int *grid_out, hipStream_t s)
{
    TileArgs a{};
    a.W = m.W;
    a.scale = m.scale;
    a.N = m.N;
    a.K = m.K;
    a.B = m.B;
    a.A = m.A;
    a.logits = m.logits;
    a.partials = m.partials;
    a.tile_ctr = m.tile_ctr;
    if (!a.tile_ctr)
        return hipErrorInvalidValue;
    const int tiles = (a.N + 15) / 16;
    int grid = device_cu_count();
    if (grid > tiles)
        grid = tiles;
    if (grid > kMaxHeadBlocks)
        grid = kMaxHeadBlocks;
    if (grid < 1)
        grid = 1;
    *grid_out = grid;
    const int seg = (a.K * (fp8 ? 1 : 2) + 1023) / 1024;  // segments per wave slice
    if (fp8) {
        if (seg <= 2)
            return launch_tile<TILE_HEAD, true, 2, 1>(a, grid, s);
        if (seg <= 4)
            return launch_tile<TILE_HEAD, true, 4, 1>(a, grid, s);
        return launch_tile<TILE_HEAD, true, 6, 1>(a, grid, s);
    }
    if (seg <= 2)
        return launch_tile<TILE_HEAD, false, 2, 1>(a, grid, s);
    if (seg <= 4)
        return launch_tile<TILE_HEAD, false, 4, 1>(a, grid, s);
    if (seg <= 6)
        return launch_tile<TILE_HEAD, false, 6, 1>(a, grid, s);
    if (seg <= 8)
        return launch_tile<TILE_HEAD, false, 4, 2>(a, grid, s);
    return launch_tile<TILE_HEAD, false, 6, 2>(a, grid, s);
}

// Whether the front tile kernel serves this shape: 2 <= B <= 16, H a multiple
// of 1024 up to 6144 (a wave's slice of a K split is H / 8 bytes, 1-6 whole
// segments), and the workspace's partial sums hold its four splits.
bool front_tile_fits(int B, int H)
{
    return B >= 2 && B <= 16 && H % 1024 == 0 && H <= 6144 &&
           eh_split(H).S >= kFrontSplits && device_cu_count() >= kFrontSplits;
}

int front_tile_splits() { return kFrontSplits; }

// eh_proj with the gather and both norms for 2 <= B <= 16: 4 K splits, one
// workgroup per CU (a multiple of 4), partial sums to P[split][b][row].
hipError_t launch_front_tile(const FrontArgs &f, const uint16_t *eh_proj, float *P, int batch,
                             hipStream_t s)
{
    TileArgs a{};
    a.W = eh_proj;
    a.N = f.H;
    a.K = 2 * f.H;
    a.B = batch;
    a.embed = f.embed;
    a.vocab = f.vocab;
    a.tokens = f.tokens;
    a.hidden = f.hidden;
    a.enorm_w = f.enorm_w;
    a.hnorm_w = f.hnorm_w;
    a.eps = f.eps;
    a.out_f32 = P;
    const int units = kFrontSplits * (f.H / 16);
    int grid = device_cu_count();
    if (grid > units)
        grid = units;
    grid -= grid % kFrontSplits;
    switch (f.H / 1024) {
    case 1: return launch_tile<TILE_FRONT, false, 1, 1>(a, grid, s);
    case 2: return launch_tile<TILE_FRONT, false, 2, 1>(a, grid, s);
    case 3: return launch_tile<TILE_FRONT, false, 3, 1>(a, grid, s);
    case 4: return launch_tile<TILE_FRONT, false, 4, 1>(a, grid, s);
    case 5: return launch_tile<TILE_FRONT, false, 5, 1>(a, grid, s);
    default: return launch_tile<TILE_FRONT, false, 6, 1>(a, grid, s);
    }
}

}  // namespace mtp
