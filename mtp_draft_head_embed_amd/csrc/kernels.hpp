// kernels.hpp -- internal launch interface between the C ABI (abi.hip) and the
// kernels.  Not part of the public header.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.hpp"

namespace mtp {

enum { PRO_FRONT = 0, PRO_HEADNORM = 1 };
enum { EPI_STORE = 0, EPI_ARGMAX = 1 };

struct RowGemvArgs {
    const void *W;        // [N][K] BF16, or E4M3FN codes for the FP8 head
    const float *scale;   // [N] per-row scale (FP8 head only)
    int N, K;
    int contig_rows;      // 0: rows dealt round-robin to waves; > 0: per-wave row blocks
    // PRO_FRONT inputs (K = 2H)
    const uint16_t *embed;
    int vocab;
    const uint32_t *tokens;
    const uint16_t *hidden;
    const uint16_t *enorm_w, *hnorm_w;
    // PRO_HEADNORM inputs (K = H)
    const uint16_t *xin;
    const uint16_t *norm_w;
    float eps;
    // outputs
    uint16_t *out;        // EPI_STORE: [B][N] BF16
    uint16_t *logits;     // EPI_ARGMAX: [B][N] BF16 or null
    Partial *partials;    // EPI_ARGMAX: [B][kMaxHeadBlocks]
    uint32_t *draft;      // EPI_ARGMAX: [B] argmax, or MTP_DRAFT_INVALID
    // EPI_ARGMAX, one sequence: kRowPools counters kCtrStride bytes apart, zero
    // at launch, that the last passes of rows are dealt from; null: every row
    // dealt round-robin
    uint32_t *row_ctr;
    // PRO_FRONT: when not null, the kRowPools counters of the head launched
    // next, set to zero
    uint32_t *zero_ctr;
};

// Batched (B >= 2) GEMM on MFMA: Y[b][n] = sum_k A[b][k] W[n][k].
struct MfmaArgs {
    const void *W;        // [N][K] BF16, or E4M3FN codes (lm_head FP8 copy)
    const float *scale;   // [N] per-row scale (FP8 head)
    int N, K;
    const uint16_t *A;    // [B][K] BF16 activations
    int B;
    int Ks;               // K columns per split (grid.y splits)
    int KC;               // K columns per LDS chunk (set by the launcher)
    int xs_off;           // LDS byte offset of the per-wave 2 KiB exchange scratch (launcher)
    int spread;           // head: deal 16-row tiles across workgroups first (launcher)
    float *out_f32;       // EPI_STORE: [splits][B][N] FP32 partial sums
    uint16_t *logits;     // EPI_ARGMAX: [B][N] BF16 or null
    Partial *partials;    // EPI_ARGMAX: [B][kMaxHeadBlocks]
    uint32_t *tile_ctr;   // EPI_ARGMAX: the tile head's kTilePools counters, zero at launch (sum_norm clears them)
};

// eh_proj K-split for the batched path: S splits of Ks columns.
struct EhSplit {
    int S, Ks;
};
EhSplit eh_split(int hidden);

struct FrontArgs {
    const uint16_t *embed;
    int vocab, H;
    const uint32_t *tokens;
    const uint16_t *hidden;
    const uint16_t *enorm_w, *hnorm_w;
    float eps;
    uint16_t *concat;     // [B][2H]
};

struct SumNormArgs {
    const float *P;       // [S][B][H] eh_proj partial sums (S > 0), or
    int S, B, H;
    const uint16_t *x_in; // [B][H] block output (S == 0)
    uint16_t *x_out;      // [B][H] BF16 x, or null
    const uint16_t *norm_w;
    float eps;
    uint16_t *xn_out;     // [B][H] BF16 normed x, or null
    uint32_t *zero_ctr;   // when not null: the tile counters of the head launched next, set to zero
};

int device_cu_count();

// eh_proj with the fused gather + dual norm prologue.
hipError_t launch_eh_proj(const RowGemvArgs &a, int batch, hipStream_t s);
// lm_head sweep with the fused head norm and argmax partials, then the
// second argmax stage (two launches).
hipError_t launch_head(const RowGemvArgs &a, bool fp8, int batch, hipStream_t s);

hipError_t launch_quantize(const uint16_t *L, int V, int H, uint8_t *q, float *scale,
                           uint32_t *flag, hipStream_t s);

hipError_t launch_front_concat(const FrontArgs &a, int batch, hipStream_t s);
hipError_t launch_sum_norm(const SumNormArgs &a, int batch, hipStream_t s);
hipError_t launch_eh_proj_mfma(const MfmaArgs &a, hipStream_t s);
hipError_t launch_head_mfma(const MfmaArgs &a, bool fp8, int *grid_out, hipStream_t s);
// lm_head for 2 <= B <= 16 at H <= 6144: one 16-row tile per workgroup at a
// time, K split over its waves (tile_gemm.hip).
bool head_tile_fits(int B, int K, bool fp8);
hipError_t launch_head_tile(const MfmaArgs &a, bool fp8, int *grid_out, hipStream_t s);
// eh_proj with the gather and both norms for 2 <= B <= 16 at H a multiple of
// 1024 up to 6144: partial sums of front_tile_splits() K splits to
// P[split][b][row] (tile_gemm.hip).
bool front_tile_fits(int B, int H);
int front_tile_splits();
hipError_t launch_front_tile(const FrontArgs &f, const uint16_t *eh_proj, float *P, int batch,
                             hipStream_t s);
hipError_t launch_argmax_final(const Partial *partials, int nparts, const uint32_t *tokens,
                               int vocab, uint32_t *draft, int batch, hipStream_t s);

}  // namespace mtp
