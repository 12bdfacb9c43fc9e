// abi.hip -- the extern "C" entry points declared in include/mtp_draft.h.
//
// Host side only: argument validation (every host-visible error is returned
// before anything is enqueued), workspace carving and kernel launches.  The
// only state kept between calls is the device address of the static scratch
// of mtp_draft_static, per GPU.
#include <mutex>

#include "../../include/mtp_draft.h"
#include "common.hpp"
#include "kernels.hpp"
#include "ctx_gemm.hpp"

using namespace mtp;

// Scratch of the allocation-free entry point (mtp_draft_static): the sweep's
// workspace in a static device array, one copy per GPU the library runs on.
// In host code this name stands for a host-side placeholder, not a device
// address; only the address hipGetSymbolAddress returns may be handed to
// kernels or runtime calls.
static __device__ __align__(256) unsigned char scratch[MTP_STATIC_SCRATCH_BYTES];

namespace {

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_shape(int32_t hidden, int32_t vocab, int32_t batch)
{
    if (hidden < 16 || hidden > MTP_MAX_HIDDEN || (hidden % 16) != 0)
        return MTP_ERR_SHAPE;
    if (vocab < 1 || vocab > MTP_MAX_VOCAB)
        return MTP_ERR_SHAPE;
    if (batch < 1 || batch > MTP_MAX_BATCH)
        return MTP_ERR_SHAPE;
    return MTP_OK;
}

// Every pointer in the list must be non-NULL and 16-byte aligned.
int check_ptrs(std::initializer_list<const void *> ps)
{
    for (const void *p : ps)
        if (!p)
            return MTP_ERR_NULL;
    for (const void *p : ps)
        if (!aligned16(p))
            return MTP_ERR_ALIGN;
    return MTP_OK;
}

int check_opt_ptr(const void *p) { return (p && !aligned16(p)) ? MTP_ERR_ALIGN : MTP_OK; }

int check_ws(const void *ws, size_t ws_bytes, int32_t hidden, int32_t batch)
{
    if (!ws)
        return MTP_ERR_WORKSPACE;
    if (!aligned16(ws))
        return MTP_ERR_ALIGN;
    if (ws_bytes < ws_layout(hidden, batch).total)
        return MTP_ERR_WORKSPACE;
    return MTP_OK;
}

#define MTP_TRY(expr)                 \
    do {                              \
        const int _rc = (expr);       \
        if (_rc != MTP_OK)            \
            return _rc;               \
    } while (0)

int validate_front(const mtp_weights *w, int32_t batch, const uint32_t *tokens, const void *hidden,
                   const void *x)
{
    if (!w)
        return MTP_ERR_NULL;
    MTP_TRY(check_shape(w->hidden, w->vocab, batch));
    MTP_TRY(check_ptrs({w->embed, w->enorm_w, w->hnorm_w, w->eh_proj, tokens, hidden, x}));
    return MTP_OK;
}

int validate_head(const mtp_weights *w, bool fp8, const uint8_t *q, const float *scale,
                  int32_t batch, const void *x, const uint32_t *draft, const void *logits)
{
    if (!w)
        return MTP_ERR_NULL;
    MTP_TRY(check_shape(w->hidden, w->vocab, batch));
    if (fp8)
        MTP_TRY(check_ptrs({w->head_norm_w, q, scale, x, draft}));
    else
        MTP_TRY(check_ptrs({w->head_norm_w, w->lm_head, x, draft}));
    MTP_TRY(check_opt_ptr(logits));
    return MTP_OK;
}

int validate_draft(const mtp_weights *w, bool fp8, const uint8_t *q, const float *scale,
                   int32_t batch, const uint32_t *tokens, const void *hidden, const uint32_t *draft,
                   const void *logits, const void *ws, size_t ws_bytes)
{
    if (!w)
        return MTP_ERR_NULL;
    MTP_TRY(check_shape(w->hidden, w->vocab, batch));
    MTP_TRY(check_ptrs({w->embed, w->enorm_w, w->hnorm_w, w->eh_proj, w->head_norm_w, tokens,
                        hidden, draft}));
    if (fp8)
        MTP_TRY(check_ptrs({q, scale}));
    else
        MTP_TRY(check_ptrs({w->lm_head}));
    MTP_TRY(check_opt_ptr(logits));
    MTP_TRY(check_ws(ws, ws_bytes, w->hidden, batch));
    return MTP_OK;
}

RowGemvArgs front_args(const mtp_weights *w, const uint32_t *tokens, const void *hidden, void *x)
{
    RowGemvArgs a{};
    a.W = w->eh_proj;
    a.N = w->hidden;
    a.K = 2 * w->hidden;
    a.embed = static_cast<const uint16_t *>(w->embed);
    a.vocab = w->vocab;
    a.tokens = tokens;
    a.hidden = static_cast<const uint16_t *>(hidden);
    a.enorm_w = static_cast<const uint16_t *>(w->enorm_w);
    a.hnorm_w = static_cast<const uint16_t *>(w->hnorm_w);
    a.eps = w->rms_eps;
    a.out = static_cast<uint16_t *>(x);
    return a;
}

char *ws_at(void *ws, size_t off) { return static_cast<char *>(ws) + off; }

// Batched front half: eh_proj over the concat rows with split-K partial sums,
// then x = BF16(sum of splits) and, when xn is wanted, the head norm of x.
// For 2 <= B <= 16 at H a multiple of 1024 up to 6144 one kernel gathers,
// normalises and multiplies (4 splits); otherwise the concat rows are written
// first and eh_proj runs on the split-K MFMA kernel.
int run_front_batched(const mtp_weights *w, int32_t batch, const uint32_t *tokens,
                      const void *hidden, void *x, void *xn, void *ws, hipStream_t s)
{
    const WsLayout L = ws_layout(w->hidden, batch);
    const int H = w->hidden;
    FrontArgs f{};
    f.embed = static_cast<const uint16_t *>(w->embed);
    f.vocab = w->vocab;
    f.H = H;
    f.tokens = tokens;
    f.hidden = static_cast<const uint16_t *>(hidden);
    f.enorm_w = static_cast<const uint16_t *>(w->enorm_w);
    f.hnorm_w = static_cast<const uint16_t *>(w->hnorm_w);
    f.eps = w->rms_eps;
    float *P = reinterpret_cast<float *>(ws_at(ws, L.p_off));
    int splits;
    if (front_tile_fits(batch, H)) {
        if (launch_front_tile(f, static_cast<const uint16_t *>(w->eh_proj), P, batch, s) !=
            hipSuccess)
            return MTP_ERR_HIP;
        splits = front_tile_splits();
    } else {
        f.concat = reinterpret_cast<uint16_t *>(ws_at(ws, L.concat_off));
        if (launch_front_concat(f, batch, s) != hipSuccess)
            return MTP_ERR_HIP;
        MfmaArgs m{};
        m.W = w->eh_proj;
        m.N = H;
        m.K = 2 * H;
        m.A = f.concat;
        m.B = batch;
        m.out_f32 = P;
        if (launch_eh_proj_mfma(m, s) != hipSuccess)
            return MTP_ERR_HIP;
        splits = eh_split(H).S;
    }
    SumNormArgs r{};
    r.P = P;
    r.S = splits;
    r.B = batch;
    r.H = H;
    r.x_out = static_cast<uint16_t *>(x);
    r.norm_w = static_cast<const uint16_t *>(w->head_norm_w);
    r.eps = w->rms_eps;
    r.xn_out = static_cast<uint16_t *>(xn);
    r.zero_ctr = reinterpret_cast<uint32_t *>(ws_at(ws, L.ctr_off));
    if (launch_sum_norm(r, batch, s) != hipSuccess)
        return MTP_ERR_HIP;
    return MTP_OK;
}

// Batched head: lm_head on MFMA over the normed xn, then the final argmax.
// Always launched right after a sum_norm on the same stream, which clears the
// head's tile counters in the workspace.
int run_head_batched(const mtp_weights *w, bool fp8, const uint8_t *q, const float *scale,
                     int32_t batch, const void *xn, const uint32_t *tokens, uint32_t *draft,
                     void *logits, void *ws, hipStream_t s)
{
    const WsLayout L = ws_layout(w->hidden, batch);
    MfmaArgs m{};
    m.W = fp8 ? static_cast<const void *>(q) : w->lm_head;
    m.scale = scale;
    m.N = w->vocab;
    m.K = w->hidden;
    m.A = static_cast<const uint16_t *>(xn);
    m.B = batch;
    m.logits = static_cast<uint16_t *>(logits);
    m.partials = reinterpret_cast<Partial *>(ws_at(ws, L.part_off));
    m.tile_ctr = reinterpret_cast<uint32_t *>(ws_at(ws, L.ctr_off));  // cleared by sum_norm
    int grid = 0;
    if (launch_head_mfma(m, fp8, &grid, s) != hipSuccess)
        return MTP_ERR_HIP;
    if (launch_argmax_final(m.partials, grid, tokens, w->vocab, draft, batch, s) != hipSuccess)
        return MTP_ERR_HIP;
    return MTP_OK;
}

// The head sweep from a block output x: norm, lm_head, argmax.  row_ctr (one
// sequence): the workspace's row counters, cleared by the eh_proj launched
// just before; null deals every row round-robin.
int run_head(const mtp_weights *w, bool fp8, const uint8_t *q, const float *scale, int32_t batch,
             const void *x, const uint32_t *tokens, uint32_t *draft, void *logits, void *ws,
             hipStream_t s, uint32_t *row_ctr = nullptr)
{
    const WsLayout L = ws_layout(w->hidden, batch);
    if (batch > 1) {
        SumNormArgs r{};
        r.S = 0;
        r.B = batch;
        r.H = w->hidden;
        r.x_in = static_cast<const uint16_t *>(x);
        r.norm_w = static_cast<const uint16_t *>(w->head_norm_w);
        r.eps = w->rms_eps;
        r.xn_out = reinterpret_cast<uint16_t *>(ws_at(ws, L.xn_off));
        r.zero_ctr = reinterpret_cast<uint32_t *>(ws_at(ws, L.ctr_off));
        if (launch_sum_norm(r, batch, s) != hipSuccess)
            return MTP_ERR_HIP;
        return run_head_batched(w, fp8, q, scale, batch, r.xn_out, tokens, draft, logits, ws, s);
    }
    RowGemvArgs a{};
    a.W = fp8 ? static_cast<const void *>(q) : w->lm_head;
    a.scale = scale;
    a.N = w->vocab;
    a.K = w->hidden;
    a.vocab = w->vocab;
    a.tokens = tokens;
    a.xin = static_cast<const uint16_t *>(x);
    a.norm_w = static_cast<const uint16_t *>(w->head_norm_w);
    a.eps = w->rms_eps;
    a.logits = static_cast<uint16_t *>(logits);
    a.partials = reinterpret_cast<Partial *>(ws_at(ws, L.part_off));
    a.draft = draft;
    a.row_ctr = row_ctr;
    if (launch_head(a, fp8, batch, s) != hipSuccess)
        return MTP_ERR_HIP;
    return MTP_OK;
}

// One whole sweep (arguments already validated), writing the block output to x.
int run_sweep(const mtp_weights *w, bool fp8, const uint8_t *q, const float *scale,
              int32_t batch, const uint32_t *tokens, const void *hidden, void *x,
              uint32_t *draft, void *logits, void *ws, hipStream_t s)
{
    const WsLayout L = ws_layout(w->hidden, batch);
    if (batch > 1) {
        void *xn = ws_at(ws, L.xn_off);
        MTP_TRY(run_front_batched(w, batch, tokens, hidden, x, xn, ws, s));
        return run_head_batched(w, fp8, q, scale, batch, xn, tokens, draft, logits, ws, s);
    }
    uint32_t *ctr = reinterpret_cast<uint32_t *>(ws_at(ws, L.ctr_off));
    RowGemvArgs f = front_args(w, tokens, hidden, x);
    f.zero_ctr = ctr;  // the head's row counters, cleared for it
    if (launch_eh_proj(f, batch, s) != hipSuccess)
        return MTP_ERR_HIP;
    return run_head(w, fp8, q, scale, batch, x, tokens, draft, logits, ws, s, ctr);
}

int run_draft(const mtp_weights *w, bool fp8, const uint8_t *q, const float *scale,
              int32_t batch, const uint32_t *tokens, const void *hidden, uint32_t *draft,
              void *logits, void *ws, size_t ws_bytes, void *stream)
{
    MTP_TRY(validate_draft(w, fp8, q, scale, batch, tokens, hidden, draft, logits, ws, ws_bytes));
    const WsLayout L = ws_layout(w->hidden, batch);
    return run_sweep(w, fp8, q, scale, batch, tokens, hidden, ws_at(ws, L.x_off), draft, logits,
                     ws, static_cast<hipStream_t>(stream));
}

// Chained drafts: workspace = the sweep's, then two block outputs used in turn.
size_t chain_ws_bytes(int32_t hidden, int32_t batch)
{
    return ws_layout(hidden, batch).total + 2 * align256(size_t(batch) * size_t(hidden) * 2);
}

int run_chain(const mtp_weights *w, bool fp8, const uint8_t *q, const float *scale,
              int32_t steps, int32_t batch, const uint32_t *tokens, const void *hidden,
              uint32_t *drafts, void *logits, void *ws, size_t ws_bytes, void *stream)
{
    if (steps < 1 || steps > MTP_MAX_CHAIN_STEPS)
        return MTP_ERR_SHAPE;
    // the first step's arguments carry every check the later steps need
    MTP_TRY(validate_draft(w, fp8, q, scale, batch, tokens, hidden, drafts, logits, ws, ws_bytes));
    if (ws_bytes < chain_ws_bytes(w->hidden, batch))
        return MTP_ERR_WORKSPACE;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const size_t base = ws_layout(w->hidden, batch).total;
    void *xbuf[2] = {ws_at(ws, base),
                     ws_at(ws, base + align256(size_t(batch) * size_t(w->hidden) * 2))};
    const size_t lrow = size_t(batch) * size_t(w->vocab) * 2;  // logits bytes per step
    for (int k = 0; k < steps; ++k) {
        const uint32_t *tk = k == 0 ? tokens : drafts + size_t(k - 1) * batch;
        const void *hd = k == 0 ? hidden : xbuf[(k - 1) & 1];
        void *lg = logits ? static_cast<void *>(static_cast<char *>(logits) + size_t(k) * lrow)
                          : nullptr;
        MTP_TRY(run_sweep(w, fp8, q, scale, batch, tk, hd, xbuf[k & 1],
                          drafts + size_t(k) * batch, lg, ws, s));
    }
    return MTP_OK;
}

// The device address of `scratch` on `dev`, resolved on the first call for
// that device with the device current (each GPU holds its own copy), then
// kept.  MTP_ERR_HIP when the runtime cannot resolve it.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch[kMaxDevices] = {};

int static_scratch(int dev, void **out)
{
    if (dev < 0 || dev >= kMaxDevices)
        return MTP_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[dev]) {
        int cur = 0;
        if (hipGetDevice(&cur) != hipSuccess)
            return MTP_ERR_HIP;
        if (cur != dev && hipSetDevice(dev) != hipSuccess)
            return MTP_ERR_HIP;
        void *p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != dev && hipSetDevice(cur) != hipSuccess)
            return MTP_ERR_HIP;
        if (e != hipSuccess || !p)
            return MTP_ERR_HIP;
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return MTP_OK;
}

}  // namespace

extern "C" {

size_t mtp_workspace_bytes(int32_t hidden, int32_t vocab, int32_t batch)
{
    if (check_shape(hidden, vocab, batch) != MTP_OK)
        return 0;
    return ws_layout(hidden, batch).total;
}

int mtp_validate_draft_args(const mtp_weights *w, int fp8, const uint8_t *q, const float *scale,
                            int32_t batch, const uint32_t *tokens, const void *hidden,
                            const uint32_t *draft, const void *logits, const void *workspace,
                            size_t ws_bytes)
{
    return validate_draft(w, fp8 != 0, q, scale, batch, tokens, hidden, draft, logits, workspace,
                          ws_bytes);
}

int mtp_quantize_head_fp8(const void *lm_head_bf16, int32_t vocab, int32_t hidden, uint8_t *q,
                          float *scale, void *workspace, size_t ws_bytes, void *stream)
{
    MTP_TRY(check_shape(hidden, vocab, 1));
    MTP_TRY(check_ptrs({lm_head_bf16, q, scale}));
    if (!workspace || ws_bytes < 256)
        return MTP_ERR_WORKSPACE;
    if (!aligned16(workspace))
        return MTP_ERR_ALIGN;
    hipStream_t s = static_cast<hipStream_t>(stream);
    uint32_t *flag = static_cast<uint32_t *>(workspace);
    if (launch_quantize(static_cast<const uint16_t *>(lm_head_bf16), vocab, hidden, q, scale, flag,
                        s) != hipSuccess)
        return MTP_ERR_HIP;
    uint32_t h_flag = 0;
    if (hipMemcpyAsync(&h_flag, flag, sizeof h_flag, hipMemcpyDeviceToHost, s) != hipSuccess)
        return MTP_ERR_HIP;
    if (hipStreamSynchronize(s) != hipSuccess)
        return MTP_ERR_HIP;
    return h_flag ? MTP_ERR_NONFINITE : MTP_OK;
}

int mtp_draft_bf16(const mtp_weights *w, int32_t batch, const uint32_t *tokens,
                   const void *hidden, uint32_t *draft, void *logits, void *workspace,
                   size_t ws_bytes, void *stream)
{
    return run_draft(w, false, nullptr, nullptr, batch, tokens, hidden, draft, logits, workspace,
                     ws_bytes, stream);
}

int mtp_draft_fp8w(const mtp_weights *w, const uint8_t *q, const float *scale, int32_t batch,
                   const uint32_t *tokens, const void *hidden, uint32_t *draft, void *logits,
                   void *workspace, size_t ws_bytes, void *stream)
{
    return run_draft(w, true, q, scale, batch, tokens, hidden, draft, logits, workspace, ws_bytes,
                     stream);
}

int mtp_draft_static(const mtp_weights *w, const uint8_t *q, const float *scale, int32_t batch,
                     const uint32_t *tokens, const void *hidden, uint32_t *draft, void *logits,
                     void *stream)
{
    if (!w)
        return MTP_ERR_NULL;
    if ((q == nullptr) != (scale == nullptr))
        return MTP_ERR_NULL;
    const bool fp8 = q != nullptr;
    MTP_TRY(check_shape(w->hidden, w->vocab, batch));
    if (ws_layout(w->hidden, batch).total > MTP_STATIC_SCRATCH_BYTES)
        return MTP_ERR_SCRATCH;
    // every other argument is checked as for the draft calls; the scratch
    // stands in for the workspace (a placeholder address: nothing is read)
    MTP_TRY(validate_draft(w, fp8, q, scale, batch, tokens, hidden, draft, logits,
                           reinterpret_cast<void *>(uintptr_t(256)), MTP_STATIC_SCRATCH_BYTES));
    hipStream_t s = static_cast<hipStream_t>(stream);
    int dev = 0;
    if (s ? hipStreamGetDevice(s, &dev) != hipSuccess : hipGetDevice(&dev) != hipSuccess)
        return MTP_ERR_HIP;
    void *ws = nullptr;
    MTP_TRY(static_scratch(dev, &ws));
    const WsLayout L = ws_layout(w->hidden, batch);
    return run_sweep(w, fp8, q, scale, batch, tokens, hidden, ws_at(ws, L.x_off), draft, logits,
                     ws, s);
}

size_t mtp_chain_workspace_bytes(int32_t hidden, int32_t vocab, int32_t batch)
{
    if (check_shape(hidden, vocab, batch) != MTP_OK)
        return 0;
    return chain_ws_bytes(hidden, batch);
}

int mtp_draft_chain_bf16(const mtp_weights *w, int32_t steps, int32_t batch,
                         const uint32_t *tokens, const void *hidden, uint32_t *drafts,
                         void *logits, void *workspace, size_t ws_bytes, void *stream)
{
    return run_chain(w, false, nullptr, nullptr, steps, batch, tokens, hidden, drafts, logits,
                     workspace, ws_bytes, stream);
}

int mtp_draft_chain_fp8w(const mtp_weights *w, const uint8_t *q, const float *scale,
                         int32_t steps, int32_t batch, const uint32_t *tokens, const void *hidden,
                         uint32_t *drafts, void *logits, void *workspace, size_t ws_bytes,
                         void *stream)
{
    return run_chain(w, true, q, scale, steps, batch, tokens, hidden, drafts, logits, workspace,
                     ws_bytes, stream);
}

int mtp_front(const mtp_weights *w, int32_t batch, const uint32_t *tokens, const void *hidden,
              void *x, void *workspace, size_t ws_bytes, void *stream)
{
    MTP_TRY(validate_front(w, batch, tokens, hidden, x));
    MTP_TRY(check_ws(workspace, ws_bytes, w->hidden, batch));
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (batch > 1)
        return run_front_batched(w, batch, tokens, hidden, x, nullptr, workspace, s);
    if (launch_eh_proj(front_args(w, tokens, hidden, x), batch, s) != hipSuccess)
        return MTP_ERR_HIP;
    return MTP_OK;
}

int mtp_head_bf16(const mtp_weights *w, int32_t batch, const void *x, uint32_t *draft,
                  void *logits, void *workspace, size_t ws_bytes, void *stream)
{
    MTP_TRY(validate_head(w, false, nullptr, nullptr, batch, x, draft, logits));
    MTP_TRY(check_ws(workspace, ws_bytes, w->hidden, batch));
    return run_head(w, false, nullptr, nullptr, batch, x, nullptr, draft, logits, workspace,
                    static_cast<hipStream_t>(stream));
}

int mtp_head_fp8w(const mtp_weights *w, const uint8_t *q, const float *scale, int32_t batch,
                  const void *x, uint32_t *draft, void *logits, void *workspace,
                  size_t ws_bytes, void *stream)
{
    MTP_TRY(validate_head(w, true, q, scale, batch, x, draft, logits));
    MTP_TRY(check_ws(workspace, ws_bytes, w->hidden, batch));
    return run_head(w, true, q, scale, batch, x, nullptr, draft, logits, workspace,
                    static_cast<hipStream_t>(stream));
}

size_t mtp_context_workspace_bytes(int32_t hidden, int32_t rows)
{
    if (check_shape(hidden, 1, 1) != MTP_OK || rows < 1 || rows > MTP_MAX_CONTEXT_ROWS)
        return 0;
    if (rows < kCtxGemmMinRows)
        return ws_layout(hidden, rows).total;
    const CtxSplit sp = ctx_split(rows, hidden, 2 * hidden);
    const size_t th = size_t(rows) * size_t(hidden);
    size_t total = align256(th * 4);  // concat [T][2H] BF16
    if (sp.S > 1)
        total += align256(size_t(sp.S) * th * 4);  // FP32 partials [S][T][H]
    return total;
}

int mtp_context_rows(const mtp_weights *w, int32_t rows, const uint32_t *tokens,
                     const void *hiddens, void *x, void *workspace, size_t ws_bytes, void *stream)
{
    if (!w)
        return MTP_ERR_NULL;
    MTP_TRY(check_shape(w->hidden, w->vocab, 1));
    if (rows < 1 || rows > MTP_MAX_CONTEXT_ROWS)
        return MTP_ERR_SHAPE;
    MTP_TRY(check_ptrs({w->embed, w->enorm_w, w->hnorm_w, w->eh_proj, tokens, hiddens, x}));
    if (!workspace)
        return MTP_ERR_WORKSPACE;
    if (!aligned16(workspace))
        return MTP_ERR_ALIGN;
    if (ws_bytes < mtp_context_workspace_bytes(w->hidden, rows))
        return MTP_ERR_WORKSPACE;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const uint32_t *tok1 = tokens + 1;  // row r pairs tokens[r + 1] with hiddens[r]
    if (rows == 1) {
        if (launch_eh_proj(front_args(w, tok1, hiddens, x), 1, s) != hipSuccess)
            return MTP_ERR_HIP;
        return MTP_OK;
    }
    if (rows < kCtxGemmMinRows)
        return run_front_batched(w, rows, tok1, hiddens, x, nullptr, workspace, s);
    const int H = w->hidden;
    FrontArgs f{};
    f.embed = static_cast<const uint16_t *>(w->embed);
    f.vocab = w->vocab;
    f.H = H;
    f.tokens = tok1;
    f.hidden = static_cast<const uint16_t *>(hiddens);
    f.enorm_w = static_cast<const uint16_t *>(w->enorm_w);
    f.hnorm_w = static_cast<const uint16_t *>(w->hnorm_w);
    f.eps = w->rms_eps;
    f.concat = static_cast<uint16_t *>(workspace);
    if (launch_front_concat(f, rows, s) != hipSuccess)
        return MTP_ERR_HIP;
    const CtxSplit sp = ctx_split(rows, H, 2 * H);
    float *P = reinterpret_cast<float *>(
        ws_at(workspace, align256(size_t(rows) * size_t(H) * 4)));
    if (launch_ctx_gemm(f.concat, static_cast<const uint16_t *>(w->eh_proj),
                        static_cast<uint16_t *>(x), P, rows, H, 2 * H, sp, s) != hipSuccess)
        return MTP_ERR_HIP;
    if (sp.S > 1) {
        SumNormArgs r{};
        r.P = P;
        r.S = sp.S;
        r.B = rows;
        r.H = H;
        r.x_out = static_cast<uint16_t *>(x);
        if (launch_sum_norm(r, rows, s) != hipSuccess)
            return MTP_ERR_HIP;
    }
    return MTP_OK;
}

const char *mtp_status_str(int status)
{
    switch (status) {
    case MTP_OK: return "ok";
    case MTP_ERR_NULL: return "a required pointer is NULL";
    case MTP_ERR_SHAPE: return "hidden, vocab or batch out of range";
    case MTP_ERR_ALIGN: return "a device pointer is not 16-byte aligned";
    case MTP_ERR_WORKSPACE: return "workspace missing or too small";
    case MTP_ERR_NONFINITE: return "a weight is NaN or Inf";
    case MTP_ERR_HIP: return "HIP runtime error";
    case MTP_ERR_SCRATCH: return "shape needs more than the static scratch of mtp_draft_static";
    default: return "unknown status";
    }
}

}  // extern "C"
