/*
 * mtp_draft.h -- C ABI of libmtpdraft.so: the GLM-5.3 MTP drafter's draft sweep
 * on one AMD Instinct MI355X (gfx950), batched over B independent sequences.
 *
 * What one draft computes (metrale_model_arch/glm5next_mtp_head.rs, module doc
 * and `forward_one`; norms per metrale_model_arch/glm5next_layer/mod.rs module
 * invariants):
 *
 *   e      = embed[token]                        contiguous BF16 row of [V][H]
 *   concat = [ enorm(e) | hnorm(hidden) ]        [2H], each norm x*w/rms
 *   x      = eh_proj . concat                    [H][2H] x [2H] -> [H]
 *   x      = block(x)                            identity here (the DSA + routed
 *                                                MoE block is not specified)
 *   logits = lm_head . shared_head_norm(x)       [V][H] x [H] -> [V]
 *   draft  = argmax(logits)                      u32, lowest index on ties
 *
 * with rms_norm_vanilla(x, w) = x * w / sqrt(mean(x^2) + eps) (never 1 + w).
 * Every intermediate the pages keep in BF16 scratch (concat, x, the normed x,
 * logits) is rounded to BF16 (round to nearest even); sums accumulate in FP32.
 * The FP8 path reads an OCP E4M3FN copy of lm_head with one f32 scale per row
 * (`head_fp8` field doc: a drafting-only copy that can change which draft is
 * proposed, never an emitted token).
 *
 * Conventions for every entry point:
 *  - Device pointers are HIP device addresses; the caller owns every buffer and
 *    the stream and keeps them alive until the enqueued work completes.  The
 *    library allocates, frees and retains nothing and has no mutable global
 *    state, except the static scratch of mtp_draft_static; calls on different
 *    streams need distinct workspaces.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *  - Layouts are row-major and densely packed.  Every device pointer must be
 *    16-byte aligned.
 *  - Shapes: 16 <= hidden <= MTP_MAX_HIDDEN with hidden % 16 == 0;
 *    1 <= vocab <= MTP_MAX_VOCAB; 1 <= batch <= MTP_MAX_BATCH.
 *  - Errors the host can see are returned before anything is enqueued.  A token
 *    >= vocab is not a host error: that sequence's draft is MTP_DRAFT_INVALID,
 *    its logits row is unspecified and no out-of-range row is read.
 *  - NaN or Inf in weights or activations is outside the contract (results are
 *    unspecified but every access stays in bounds).
 *  - The draft entry points are asynchronous: they enqueue kernels on `stream`
 *    and return; no host<->device copy happens.  Only mtp_quantize_head_fp8
 *    synchronises `stream` (to report non-finite weights).
 */
#ifndef MTP_DRAFT_H
#define MTP_DRAFT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes returned by every int-returning entry point. */
enum {
    MTP_OK = 0,
    MTP_ERR_NULL = 1,      /* a required pointer is NULL                        */
    MTP_ERR_SHAPE = 2,     /* hidden, vocab or batch out of range               */
    MTP_ERR_ALIGN = 3,     /* a device pointer is not 16-byte aligned           */
    MTP_ERR_WORKSPACE = 4, /* workspace NULL or smaller than mtp_workspace_bytes */
    MTP_ERR_NONFINITE = 5, /* quantiser: a weight is NaN or Inf                  */
    MTP_ERR_HIP = 6,       /* a HIP runtime call or kernel launch failed        */
    MTP_ERR_SCRATCH = 7    /* mtp_draft_static: the shape needs more than
                              MTP_STATIC_SCRATCH_BYTES of scratch              */
};

#define MTP_DRAFT_INVALID 0xFFFFFFFFu /* draft[b] when tokens[b] >= vocab */
#define MTP_MAX_HIDDEN 8192
#define MTP_MAX_VOCAB 16777216 /* 2^24 */
#define MTP_MAX_BATCH 64
#define MTP_MAX_CONTEXT_ROWS 65536
#define MTP_MAX_CHAIN_STEPS 64
#define MTP_STATIC_SCRATCH_BYTES (16u << 20) /* scratch of mtp_draft_static, per GPU */

/* The drafter's weights, all BF16 device arrays (glm5next_mtp_head.rs: the
 * head owns `embed_tokens`, the target's `lm_head`, and the MTP module's
 * enorm, hnorm, eh_proj, final norm and rms_eps). */
typedef struct mtp_weights {
    int32_t hidden;          /* H                                              */
    int32_t vocab;           /* V                                              */
    float rms_eps;           /* eps inside the square root, as f32             */
    const void *embed;       /* [V][H]   embed_tokens                          */
    const void *enorm_w;     /* [H]      norm of the embedding row             */
    const void *hnorm_w;     /* [H]      norm of the target hidden             */
    const void *head_norm_w; /* [H]      shared_head.norm                      */
    const void *eh_proj;     /* [H][2H]  input is [enorm(e) | hnorm(hidden)]    */
    const void *lm_head;     /* [V][H]   may be NULL for the FP8-only calls    */
} mtp_weights;

/* Bytes of device workspace the draft, head and front calls need for this
 * shape (0 when the shape is out of range).  The workspace holds the concat
 * vectors, the block input x and the per-workgroup argmax partials; its
 * contents on entry do not matter. */
size_t mtp_workspace_bytes(int32_t hidden, int32_t vocab, int32_t batch);

/* Host-only check of the arguments of mtp_draft_bf16 (fp8 == 0) or
 * mtp_draft_fp8w (fp8 != 0); touches no device and enqueues nothing.  Returns
 * the status the draft call would return before launching. */
int mtp_validate_draft_args(const mtp_weights *w, int fp8, const uint8_t *q, const float *scale,
                            int32_t batch, const uint32_t *tokens, const void *hidden,
                            const uint32_t *draft, const void *logits, const void *workspace,
                            size_t ws_bytes);

/* FP8 drafting copy of lm_head (glm5next_mtp_head.rs, `head_fp8` doc: an E4M3
 * copy; quantisation may fail, and the caller then keeps the BF16 head).
 * Per row v:  s[v] = amax_v / 448 (f32, correctly rounded; 1 for an all-zero
 * row), q[v][j] = E4M3FN(clamp(fl32(L[v][j] / s[v]), -448, 448)), round to
 * nearest, ties to even, sign of zero kept.
 *   lm_head_bf16  device BF16 [vocab][hidden]       (read)
 *   q             device u8   [vocab][hidden]       (written)
 *   scale         device f32  [vocab]               (written)
 *   workspace     device, >= 256 bytes               (scratch flag)
 * Synchronises `stream`.  Returns MTP_ERR_NONFINITE when any weight is NaN or
 * Inf (q and scale are then unspecified). */
int mtp_quantize_head_fp8(const void *lm_head_bf16, int32_t vocab, int32_t hidden, uint8_t *q,
                          float *scale, void *workspace, size_t ws_bytes, void *stream);

/* One draft per sequence with the BF16 lm_head (glm5next_mtp_head.rs,
 * `forward_one`, unsharded sweep).
 *   w          weights (lm_head required)
 *   batch      B
 *   tokens     device u32  [B]       token whose embedding row is read
 *   hidden     device BF16 [B][H]    target hidden paired with that token
 *   draft      device u32  [B]       (written) argmax, or MTP_DRAFT_INVALID
 *   logits     device BF16 [B][V]    (written) or NULL to skip storing them
 *   workspace  device, >= mtp_workspace_bytes(H, V, B)
 * Asynchronous on `stream`. */
int mtp_draft_bf16(const mtp_weights *w, int32_t batch, const uint32_t *tokens,
                   const void *hidden, uint32_t *draft, void *logits, void *workspace,
                   size_t ws_bytes, void *stream);

/* As mtp_draft_bf16, but the head reads the FP8 copy made by
 * mtp_quantize_head_fp8 (glm5next_mtp_head.rs, `forward_one`,
 * `dense_gemv_fp8w`): logit_v = BF16(scale[v] * sum_j dec(q[v][j]) * xn_j).
 *   q      device u8  [V][H] E4M3FN codes
 *   scale  device f32 [V]
 * w->lm_head is not read and may be NULL. */
int mtp_draft_fp8w(const mtp_weights *w, const uint8_t *q, const float *scale, int32_t batch,
                   const uint32_t *tokens, const void *hidden, uint32_t *draft, void *logits,
                   void *workspace, size_t ws_bytes, void *stream);

/* Allocation-free draft call, for callers that cannot allocate device memory
 * or pass a workspace (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  The same sweep as mtp_draft_bf16 (q and
 * scale both NULL: the BF16 lm_head) or mtp_draft_fp8w (q and scale both
 * non-NULL: the FP8 copy), with the same arguments, results and errors, minus
 * the workspace: its scratch is a static device array of
 * MTP_STATIC_SCRATCH_BYTES inside the library, one per GPU, held until the
 * process ends.  The call allocates nothing.
 *  - A shape whose workspace (mtp_workspace_bytes) exceeds
 *    MTP_STATIC_SCRATCH_BYTES returns MTP_ERR_SCRATCH before anything is
 *    enqueued; at H = 6144 every batch up to 32 fits.
 *  - Every call on one GPU shares that GPU's scratch, which keeps the last
 *    call's contents (no call needs it cleared): calls that can overlap on one
 *    GPU (different streams, or different host threads) race and must be
 *    serialised by the caller.
 *  - The first call on a GPU resolves the scratch's device address (a runtime
 *    query, no allocation); make that call outside graph capture.
 * Asynchronous on `stream`. */
int mtp_draft_static(const mtp_weights *w, const uint8_t *q, const float *scale, int32_t batch,
                     const uint32_t *tokens, const void *hidden, uint32_t *draft, void *logits,
                     void *stream);

/* The front half alone (glm5next_mtp_head.rs, `forward_one` up to the block):
 * gather, enorm, hnorm, concat and eh_proj, writing the block input
 *   x  device BF16 [B][H]  (written; row b unspecified when tokens[b] >= V)
 * Uses w->embed, enorm_w, hnorm_w, eh_proj.  Asynchronous. */
int mtp_front(const mtp_weights *w, int32_t batch, const uint32_t *tokens, const void *hidden,
              void *x, void *workspace, size_t ws_bytes, void *stream);

/* The head alone (glm5next_mtp_head.rs, `forward_one` after the block):
 * shared_head.norm of x, the BF16 lm_head sweep and the argmax.
 *   x       device BF16 [B][H]  block output (read)
 *   draft   device u32  [B]     (written)
 *   logits  device BF16 [B][V]  (written) or NULL
 * Uses w->head_norm_w and w->lm_head.  Asynchronous. */
int mtp_head_bf16(const mtp_weights *w, int32_t batch, const void *x, uint32_t *draft,
                  void *logits, void *workspace, size_t ws_bytes, void *stream);

/* The head alone with the FP8 copy (q, scale as for mtp_draft_fp8w). */
int mtp_head_fp8w(const mtp_weights *w, const uint8_t *q, const float *scale, int32_t batch,
                  const void *x, uint32_t *draft, void *logits, void *workspace,
                  size_t ws_bytes, void *stream);

/* Context rows (glm5next_mtp_head.rs, `rows_impl`): the drafter's prompt or
 * catch-up rows through the front half.  Row r pairs the embedding of
 * tokens[r + 1] with hiddens[r]:
 *   x[r] = BF16(eh_proj . [enorm(embed[tokens[r+1]]) | hnorm(hiddens[r])])
 * (the page then writes each row into the MTP block's KV cache, which is not
 * part of this library).  At many rows this is a dense GEMM on MFMA.
 *   rows       T, 1 <= T <= MTP_MAX_CONTEXT_ROWS
 *   tokens     device u32  [T + 1]   (tokens[0] is not read)
 *   hiddens    device BF16 [T][H]
 *   x          device BF16 [T][H]    (written; row r unspecified when
 *                                     tokens[r + 1] >= V)
 *   workspace  device, >= mtp_context_workspace_bytes(H, T)
 * Uses w->embed, enorm_w, hnorm_w, eh_proj.  Asynchronous. */
size_t mtp_context_workspace_bytes(int32_t hidden, int32_t rows);
int mtp_context_rows(const mtp_weights *w, int32_t rows, const uint32_t *tokens,
                     const void *hiddens, void *x, void *workspace, size_t ws_bytes,
                     void *stream);

/* Chained drafts (glm5next_mtp_head.rs: `propose` writes several drafts per
 * call -- the state's `last_drafted` -- each one a `forward_one`).  Step k + 1
 * takes step k's draft as its token and step k's block output x as its hidden;
 * the pages do not show which hidden the proposer feeds back, and with the
 * block taken as the identity x is the MTP layer's output before
 * shared_head.norm.  Equivalent to `steps` calls of mtp_draft_bf16 (or
 * mtp_draft_fp8w) with those inputs, enqueued back to back with no host
 * round trip.
 *   steps      K, 1 <= K <= MTP_MAX_CHAIN_STEPS
 *   tokens     device u32  [B]        first step's tokens
 *   hidden     device BF16 [B][H]     first step's hidden
 *   drafts     device u32  [K][B]     (written) drafts[k][b]; once a draft is
 *                                      MTP_DRAFT_INVALID, every later one of
 *                                      that sequence is too
 *   logits     device BF16 [K][B][V]  (written) or NULL
 *   workspace  device, >= mtp_chain_workspace_bytes(H, V, B)
 * Other arguments and errors as for mtp_draft_bf16 / mtp_draft_fp8w; K out of
 * range is MTP_ERR_SHAPE.  Asynchronous. */
size_t mtp_chain_workspace_bytes(int32_t hidden, int32_t vocab, int32_t batch);
int mtp_draft_chain_bf16(const mtp_weights *w, int32_t steps, int32_t batch,
                         const uint32_t *tokens, const void *hidden, uint32_t *drafts,
                         void *logits, void *workspace, size_t ws_bytes, void *stream);
int mtp_draft_chain_fp8w(const mtp_weights *w, const uint8_t *q, const float *scale,
                         int32_t steps, int32_t batch, const uint32_t *tokens, const void *hidden,
                         uint32_t *drafts, void *logits, void *workspace, size_t ws_bytes,
                         void *stream);

/* Static text for a status code. */
const char *mtp_status_str(int status);

#ifdef __cplusplus
}
#endif

#endif /* MTP_DRAFT_H */
