/*
 * mtp_probe.h -- measurement and verification aids of libmtpdraft.so, not
 * steps of the draft sweep: a plain streaming read of a device buffer (the
 * practical HBM ceiling that the weight sweeps are compared with), and a check
 * of the hardware FP32 -> E4M3FN convert that the FP8 quantiser relies on.
 */
#ifndef MTP_PROBE_H
#define MTP_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Reads `bytes` of the device buffer `buf` once with 16-byte non-temporal
 * loads (consecutive lanes on consecutive pieces, eight loads in flight per
 * lane, grid-stride), from `wg_per_cu` 256-thread workgroups per CU.
 *   buf        device, 16-byte aligned, read only
 *   bytes      a positive multiple of 16
 *   out        device u32 [1], 4-byte aligned: written only if the XOR of a
 *              lane's words equals a fixed constant (keeps the loads live)
 *   wg_per_cu  1..16
 * Asynchronous on `stream` (a hipStream_t as void*).  Returns MTP_OK,
 * MTP_ERR_NULL, MTP_ERR_SHAPE, MTP_ERR_ALIGN or MTP_ERR_HIP (mtp_draft.h). */
int mtp_probe_stream_read(const void *buf, size_t bytes, uint32_t *out, int32_t wg_per_cu,
                          void *stream);

/* Checks the gfx950 convert v_cvt_pk_fp8_f32 on every float32 x with
 * |x| <= 448 (both signs, 2 277 507 074 values) against round to nearest,
 * ties to even, onto the OCP E4M3FN codes (an integer encoder on the binary32
 * bits; subnormal codes below 2^-6).  The FP8 quantiser encodes with this
 * convert (mtp_quantize_head_fp8's codes are defined by that rounding).
 *   result  device u32 [2], 4-byte aligned: [0] values whose codes differ,
 *           [1] values checked
 * Asynchronous on `stream`.  Returns MTP_OK, MTP_ERR_NULL, MTP_ERR_ALIGN or
 * MTP_ERR_HIP. */
int mtp_probe_fp8_convert(uint32_t *result, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MTP_PROBE_H */
