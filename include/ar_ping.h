/*
 * ar_ping.h -- the one-way flag hop between two workgroups (MI355X, gfx950):
 *              the latency floor of the small AllReduce calls beside the
 *              launch floor of a graph node.
 *
 * The barrier-free AllReduce of the "微秒必争：英伟达与苏黎世联邦理工学院如何
 * 突破多GPU通信延迟极限" page replaces both global barriers of a call by flags
 * that travel with the data (section "破局之道：无屏障同步的四大核心机制"), so
 * at decode sizes a call costs at least one launch plus one flag hop from a
 * writer to its readers (section "张量并行与AllReduce：推理场景下的通信瓶颈",
 * the speed-of-light figure set against the measured call).  This entry
 * point measures that hop on the device at hand: two single-lane workgroups
 * bounce a counter through two flag words, with the AllReduce kernels' store
 * and poll policies, either inside one XCD's L2 (the layout of the XCD-local
 * kernels) or between two XCDs at device scope (the stand-in for a hop
 * between GPUs).  It is a measurement, not a step of the AllReduce.
 *
 * Conventions as in ar.h: int status (AR_OK or a negative ar_status code),
 * asynchronous on `stream`, no allocation.  It needs no ar_init.
 */
#ifndef TPDC_AR_PING_H
#define TPDC_AR_PING_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * ar_flag_ping -- `rounds` round trips of a flag between two workgroups.
 *   rounds: 1 <= rounds <= 2^20;
 *   cross_xcd: 0 = both workgroups on one XCD, stores and polls coherent in
 *     its L2; 1 = the two on XCDs next to each other in dispatch order,
 *     device-scope stores and polls (workgroups are dealt to the 8 XCDs
 *     round-robin from an offset that varies from launch to launch, so the
 *     XCDs are reported, not chosen);
 *   out: device pointer, 8-byte aligned, to 5 uint64 words the kernel writes:
 *     [0] clock ticks (100 MHz constant clock) of the whole exchange, timed by
 *         the first workgroup; one way = ticks / (2 rounds) x 10 ns;
 *     [1] the first workgroup's status, [4] the second's: 0, or 1 if a wait
 *         ran past its 200 ms budget (the kernel then ends anyway);
 *     [2], [3] the XCD each workgroup ran on (the caller checks the placement);
 *   stream: the HIP stream the kernel is enqueued on.
 * Calls on one device must not overlap (they share the two flag words).
 * Returns AR_ERR_INVALID for arguments outside this contract (nothing is
 * launched), AR_ERR_HIP if the device query or the launch fails, else AR_OK.
 */
int ar_flag_ping(uint32_t rounds, int cross_xcd, void *out, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif
