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
};

int device_cu_count();

// eh_proj with the fused gather + dual norm prologue.
hipError_t launch_eh_proj(const RowGemvArgs &a, int batch, hipStream_t s);
// lm_head sweep with the fused head norm and argmax partials, then the
// second argmax stage (two launches).
hipError_t launch_head(const RowGemvArgs &a, bool fp8, int batch, hipStream_t s);

hipError_t launch_quantize(const uint16_t *L, int V, int H, uint8_t *q, float *scale,
                           uint32_t *flag, hipStream_t s);

}  // namespace mtp
