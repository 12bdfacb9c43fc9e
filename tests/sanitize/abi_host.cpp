// Drives the host-side layer of libmtpdraft (argument validation, workspace
// sizing, status strings) over valid and invalid arguments.  Every call here
// returns before anything would be enqueued, so no GPU is needed.  Built with
// address and undefined-behaviour sanitizers on the host code by
// tests/test_sanitizers_cpu.py.
#include <cstdint>
#include <cstdio>
#include <initializer_list>

#include "../../include/mtp_draft.h"

static int fails = 0;
#define EXPECT(cond)                                                     \
    do {                                                                 \
        if (!(cond)) {                                                   \
            std::printf("failed at line %d: %s\n", __LINE__, #cond);      \
            ++fails;                                                     \
        }                                                                \
    } while (0)

static void *P(uintptr_t a) { return reinterpret_cast<void *>(a); }

int main()
{
    const int hs[] = {-16, 0, 8, 16, 24, 256, 6144, 8192, 8208, 1 << 30};
    const int vs[] = {-1, 0, 1, 4096, 154880, 1 << 24, (1 << 24) + 1, 0x7FFFFFFF};
    const int bs[] = {-1, 0, 1, 2, 16, 17, 64, 65};
    for (int h : hs)
        for (int v : vs)
            for (int b : bs) {
                const bool ok = h >= 16 && h <= 8192 && h % 16 == 0 && v >= 1 && v <= (1 << 24) &&
                                b >= 1 && b <= 64;
                EXPECT((mtp_workspace_bytes(h, v, b) > 0) == ok);
                EXPECT((mtp_chain_workspace_bytes(h, v, b) > 0) == ok);
            }
    for (int h : hs)
        for (int t : {-1, 0, 1, 16, 17, 128, 129, 4096, 65536, 65537}) {
            const bool ok = h >= 16 && h <= 8192 && h % 16 == 0 && t >= 1 && t <= 65536;
            EXPECT((mtp_context_workspace_bytes(h, t) > 0) == ok);
        }
    for (int s = -3; s < 12; ++s)
        EXPECT(mtp_status_str(s) != nullptr);

    mtp_weights w{};
    w.hidden = 64;
    w.vocab = 100;
    w.rms_eps = 1e-6f;
    w.embed = P(0x10000);
    w.enorm_w = P(0x20000);
    w.hnorm_w = P(0x30000);
    w.head_norm_w = P(0x40000);
    w.eh_proj = P(0x50000);
    w.lm_head = P(0x60000);
    const size_t ws = mtp_workspace_bytes(64, 100, 4);
    auto val = [&](const mtp_weights *pw, int fp8, int b, uintptr_t tok, uintptr_t hid,
                   uintptr_t dr, uintptr_t lg, uintptr_t wsp, size_t wsb) {
        return mtp_validate_draft_args(pw, fp8, static_cast<const uint8_t *>(P(0x70000)),
                                       static_cast<const float *>(P(0x80000)), b,
                                       static_cast<const uint32_t *>(P(tok)), P(hid),
                                       static_cast<const uint32_t *>(P(dr)), P(lg), P(wsp), wsb);
    };
    EXPECT(val(&w, 0, 4, 0x90000, 0xA0000, 0xB0000, 0, 0xC0000, ws) == MTP_OK);
    EXPECT(val(&w, 1, 4, 0x90000, 0xA0000, 0xB0000, 0xD0000, 0xC0000, ws) == MTP_OK);
    EXPECT(val(nullptr, 0, 4, 0x90000, 0xA0000, 0xB0000, 0, 0xC0000, ws) == MTP_ERR_NULL);
    EXPECT(val(&w, 0, 0, 0x90000, 0xA0000, 0xB0000, 0, 0xC0000, ws) == MTP_ERR_SHAPE);
    EXPECT(val(&w, 0, 65, 0x90000, 0xA0000, 0xB0000, 0, 0xC0000, ws) == MTP_ERR_SHAPE);
    EXPECT(val(&w, 0, 4, 0, 0xA0000, 0xB0000, 0, 0xC0000, ws) == MTP_ERR_NULL);
    EXPECT(val(&w, 0, 4, 0x90004, 0xA0000, 0xB0000, 0, 0xC0000, ws) == MTP_ERR_ALIGN);
    EXPECT(val(&w, 0, 4, 0x90000, 0xA0000, 0xB0000, 0xD0008, 0xC0000, ws) == MTP_ERR_ALIGN);
    EXPECT(val(&w, 0, 4, 0x90000, 0xA0000, 0xB0000, 0, 0, ws) == MTP_ERR_WORKSPACE);
    EXPECT(val(&w, 0, 4, 0x90000, 0xA0000, 0xB0000, 0, 0xC0000, ws - 1) == MTP_ERR_WORKSPACE);
    mtp_weights w2 = w;
    w2.lm_head = nullptr;
    EXPECT(val(&w2, 0, 4, 0x90000, 0xA0000, 0xB0000, 0, 0xC0000, ws) == MTP_ERR_NULL);
    EXPECT(val(&w2, 1, 4, 0x90000, 0xA0000, 0xB0000, 0, 0xC0000, ws) == MTP_OK);
    w2 = w;
    w2.hidden = 72;
    EXPECT(val(&w2, 0, 4, 0x90000, 0xA0000, 0xB0000, 0, 0xC0000, ws) == MTP_ERR_SHAPE);

    // the enqueueing entry points reject the same arguments before any HIP call
    const uint32_t *tk = static_cast<const uint32_t *>(P(0x90000));
    uint32_t *dr = static_cast<uint32_t *>(P(0xB0000));
    EXPECT(mtp_draft_bf16(&w, 0, tk, P(0xA0000), dr, nullptr, P(0xC0000), ws, nullptr) ==
           MTP_ERR_SHAPE);
    EXPECT(mtp_draft_fp8w(&w, nullptr, nullptr, 1, tk, P(0xA0000), dr, nullptr, P(0xC0000), ws,
                          nullptr) == MTP_ERR_NULL);
    EXPECT(mtp_front(&w, 1, tk, P(0xA0000), nullptr, P(0xC0000), ws, nullptr) == MTP_ERR_NULL);
    EXPECT(mtp_head_bf16(&w, 1, P(0xA0000), dr, nullptr, P(0xC0000), 0, nullptr) ==
           MTP_ERR_WORKSPACE);
    EXPECT(mtp_head_fp8w(&w, nullptr, nullptr, 1, P(0xA0000), dr, nullptr, P(0xC0000), ws,
                         nullptr) == MTP_ERR_NULL);
    EXPECT(mtp_context_rows(&w, 0, tk, P(0xA0000), P(0xD0000), P(0xC0000), ws, nullptr) ==
           MTP_ERR_SHAPE);
    EXPECT(mtp_context_rows(&w, 70000, tk, P(0xA0000), P(0xD0000), P(0xC0000), ws, nullptr) ==
           MTP_ERR_SHAPE);
    EXPECT(mtp_draft_chain_bf16(&w, 0, 1, tk, P(0xA0000), dr, nullptr, P(0xC0000), ws, nullptr) ==
           MTP_ERR_SHAPE);
    EXPECT(mtp_draft_chain_bf16(&w, 2, 1, tk, P(0xA0000), dr, nullptr, P(0xC0000), 16, nullptr) ==
           MTP_ERR_WORKSPACE);
    EXPECT(mtp_quantize_head_fp8(P(0x60000), 100, 60, static_cast<uint8_t *>(P(0x70000)),
                                 static_cast<float *>(P(0x80000)), P(0xC0000), 256, nullptr) ==
           MTP_ERR_SHAPE);
    EXPECT(mtp_quantize_head_fp8(P(0x60000), 100, 64, static_cast<uint8_t *>(P(0x70000)),
                                 static_cast<float *>(P(0x80000)), P(0xC0000), 255, nullptr) ==
           MTP_ERR_WORKSPACE);
    std::printf(fails ? "%d checks failed\n" : "host layer ok\n", fails);
    return fails ? 1 : 0;
}
