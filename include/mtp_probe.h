/*
 * mtp_probe.h -- a measurement aid of libmtpdraft.so, not a step of the
 * draft sweep: a plain streaming read of a device buffer, the practical HBM
 * ceiling that the weight sweeps are compared with.
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

#ifdef __cplusplus
}
#endif

#endif /* MTP_PROBE_H */
