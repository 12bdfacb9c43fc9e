// ctx_gemm.hpp -- launcher of the context-row eh_proj GEMM (ctx_gemm.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mtp {

// Context rows: C[M][N] = BF16(A[M][K] . W[N][K]^T) on MFMA in one of three
// tile shapes, with K split S ways (Ks columns each, a multiple of 128) when
// the tiles alone would leave CUs idle; then the FP32 partials P[S][M][N] are
// summed by launch_sum_norm.
enum CtxTile { kCtxTile128x128 = 1, kCtxTile256x256 = 2, kCtxTile256x192 = 3 };
struct CtxSplit {
    int S, Ks;
    int tile;  // CtxTile
};
CtxSplit ctx_split(int M, int N, int K);
hipError_t launch_ctx_gemm(const uint16_t *A, const uint16_t *W, uint16_t *C, float *P, int M,
                           int N, int K, CtxSplit sp, hipStream_t s);
// Rows from which the context rows use the tiled GEMM instead of the batched
// split-K sweep.
constexpr int kCtxGemmMinRows = 17;
// Rows from which the GEMM uses the 256 x 256 or 256 x 192 tile (whichever
// fills the CUs in fewer rounds) instead of 128 x 128: the small tile is
// faster while one row tile holds every row (eh_proj then streams once),
// the large ones from the row count where the small tile would need two.
constexpr int kCtxBigTileMinRows = 129;

}  // namespace mtp
