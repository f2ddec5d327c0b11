/*
 * ar_copy.h -- a plain device-to-device copy, the bandwidth reference that
 *              the AllReduce's bandwidth-bound sizes are read against
 *              (MI355X, gfx950).
 *
 * At its large sizes the two-shot AllReduce reads every rank's input once
 * and writes every rank's output copy once, the reduce-scatter followed by
 * the all-gather of the "微秒必争：英伟达与苏黎世联邦理工学院如何突破多GPU
 * 通信延迟极限" page (its table of one-shot and two-shot variants by message
 * size).  A copy of the same byte count has the same memory traffic and no
 * synchronisation at all, so timed back to back like the AllReduce calls it
 * measures what the device's memory delivers for that traffic at that launch
 * cadence on the machine at hand, beside the datasheet peak.  It is a
 * measurement reference, not a step of the AllReduce.
 *
 * The copy uses the launch shape of the AllReduce's bandwidth-bound data
 * phase: 256-thread workgroups (at most 512), each lane moving two 16-byte
 * vectors per round with plain loads and streaming (non-temporal) stores.
 *
 * Conventions as in ar.h: int status (AR_OK or a negative ar_status code),
 * plain device pointers owned by the caller, asynchronous on `stream`, no
 * allocation (capture-safe).  It needs no ar_init.
 */
#ifndef TPDC_AR_COPY_H
#define TPDC_AR_COPY_H

#include <stddef.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * ar_copy -- dst[0 .. bytes) = src[0 .. bytes).
 *   src, dst: device pointers, 16-byte aligned, the two ranges disjoint;
 *   bytes: a multiple of 16, 16 <= bytes <= 2^31 - 16;
 *   stream: the HIP stream the copy is enqueued on.
 * Returns AR_ERR_INVALID for arguments outside this contract (nothing is
 * launched), AR_ERR_HIP if the launch fails, else AR_OK.
 */
int ar_copy(const void *src, void *dst, size_t bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif
