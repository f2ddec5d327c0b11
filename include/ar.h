/*
 * ar.h -- barrier-free fixed-order bf16 AllReduce for tensor-parallel decode,
 *         MI355X (gfx950), C ABI.
 *
 * The operation.  Every tensor-parallel rank holds a partial result; the
 * AllReduce sums the partial results element by element and gives the full
 * sum to every rank ("Every Microsecond Counts" write-up, page "微秒必争：英伟达
 * 与苏黎世联邦理工学院如何突破多GPU通信延迟极限", section "张量并行与AllReduce").
 * Here each element's sum is a left fold over ranks 0..N-1 in IEEE binary32
 * started from rank 0's value, rounded once to bfloat16 (round to nearest,
 * ties to even); every rank's output copy holds the same bits.
 *
 * How ranks synchronise.  No global memory barrier is used (same page,
 * section "全局内存屏障": a barrier before reading and one before the next
 * overwrite).  Validity travels with the data instead (section "四大核心机制"):
 *   - LL: 8-byte units {2 bf16, 32-bit flag}; a unit whose flag equals the
 *     call's flag holds the call's data (item 1, LL);
 *   - sentinel: receive buffers are pre-filled with the bf16 NaN pattern
 *     0xFFFF; any other value is data; the receiver re-fills what it read
 *     (item 2, Sentinel; reset()/resetRange() in section "统一原语与API设计");
 *   - double buffering: a message is walked in rounds through two
 *     fixed-size staging windows per rank; round j uses window (flag of
 *     round j) & 1, and receiving round j from every peer proves each peer
 *     finished reading round j-1, so its window may be overwritten (item 3,
 *     double buffering);
 *   - LL128-style lines: 128-byte lines of 120 payload bytes and an 8-byte
 *     flag, the flag written after the payload (item 4 gives the 128-byte
 *     line; its NVLink atomic-add form has no counterpart here).
 * Algorithms (section "统一原语与API设计", table of variants): one-shot (every
 * rank reads all N contributions) below 64 KiB per rank, two-shot
 * (reduce-scatter then all-gather) above.
 *
 * Emulation.  On one GPU the N ranks are disjoint sets of workgroups of one
 * kernel launch; they exchange data only through staging buffers and flag
 * words in device memory.  Part p of every rank's work runs on one XCD
 * (the hardware deals workgroups to the 8 XCDs round-robin), so one part's
 * exchange stays inside one XCD's L2.  Staging and flag accesses are
 * device-scope coherent, or -- once ar_init has verified the round-robin
 * dispatch -- XCD-local (see ar_set_scope).
 *
 * Conventions for every entry point:
 *   - return value: AR_OK (0) or a negative ar_status code; nothing aborts;
 *   - device pointers are plain hipMalloc (or torch) allocations on the
 *     device that was current at ar_init; the caller owns them;
 *   - one process-wide context; calls come from one host thread.
 */
#ifndef TPDC_AR_H
#define TPDC_AR_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

enum ar_status {
    AR_OK = 0,
    AR_ERR_INVALID = -1,    /* an argument breaks the stated contract */
    AR_ERR_NOT_INIT = -2,   /* ar_init has not succeeded */
    AR_ERR_STATE = -3,      /* already initialised / wrong call order */
    AR_ERR_OOM = -4,        /* device allocation failed */
    AR_ERR_HIP = -5,        /* a HIP runtime call failed (see ar_last_hip_error) */
    AR_ERR_TIMEOUT = -6     /* a device poll exceeded the watchdog (ar_get_status) */
};

enum ar_scope {
    AR_SCOPE_AUTO = 0,      /* XCD-local when ar_init verified the placement and
                               the launch's part count is a multiple of 8 */
    AR_SCOPE_DEVICE = 1,    /* device scope always: correct on any placement */
    AR_SCOPE_CROSS_XCD = 2  /* device scope with rank r's workgroups on XCD r mod 8
                               (grid (1, N, parts)): every exchange between ranks on
                               different XCDs crosses L2s -- the one-GPU stand-in
                               for a hop between GPUs */
};

enum ar_algo { AR_ALGO_AUTO = 0, AR_ALGO_ONESHOT = 1, AR_ALGO_TWOSHOT = 2 };

enum ar_proto {
    AR_PROTO_AUTO = 0,
    AR_PROTO_LL = 1,        /* one-shot only */
    AR_PROTO_LL128 = 2,     /* one-shot or two-shot */
    AR_PROTO_SENTINEL = 3,  /* one-shot or two-shot */
    AR_PROTO_DIRECT = 4,    /* arrival flags instead of staging: one-shot reads
                               peers' inputs in place; two-shot reads slice q in
                               place and writes the reduced slice straight into
                               every rank's output, then completion flags */
    AR_PROTO_BARRIER = 5,   /* measured baseline, not barrier-free: the DIRECT
                               reads, fold and writes between two device-wide
                               barriers over all ranks' workgroups (before the
                               reads, after the writes), the classic structure of
                               section "全局内存屏障"; the grid stays within half the
                               device's resident-workgroup capacity */
    AR_PROTO_ATOMIC = 6     /* two-shot only: the atomic two-phase algorithm of
                               section "四大核心机制" item 4 -- every rank adds its
                               values into shared 128-byte lines {counter,
                               31 x binary32} with atomics and counts itself in;
                               a rank reads a line once its counter reaches N.
                               Sums are taken in arrival order, so the result is
                               NOT the fixed-order fold: before the bf16 rounding
                               it is within (N-1) * 2^-24 * sum_r |x_r| of the
                               exact sum, and all N copies agree */
};

#define AR_MAX_RANKS 16

/*
 * ar_init -- create the context on the current HIP device (the C ABI's
 * counterpart of the pages' NCCL-compatible drop-in: "SiFAR" page, section
 * on deployment; the operation itself: "微秒必争…", section "张量并行与
 * AllReduce").
 *   n_ranks:   number of emulated ranks, 1..16.
 *   max_elems: largest per-rank element count any later call may use, > 0,
 *              rounded up to a multiple of 8.  All n_ranks output copies of
 *              the binary32 debug path must span at most 2^31 bytes, which
 *              gives max_elems <= 2^29 / n_ranks (2^26 for 8 ranks, 128 MiB
 *              of bf16 per rank).
 * Allocates every protocol's staging: fixed-size windows per rank (LL,
 * LL128) or per (receiver, sender) inbox pair (sentinel) and buffer, of
 * min(what a max_elems message needs in one round, 1 MiB (LL, LL128) or
 * 256 KiB (sentinel)) -- larger messages walk their rounds through them
 * (ar_set_staging) -- plus the two sequence words, the status record and the
 * flag words of the arrival, completion and barrier handshakes; zeroes flag
 * words and arms sentinel buffers with 0xFFFF.  Synchronous.
 * Start-up defaults may come from the environment: AR_ALGO (auto, oneshot,
 * twoshot), AR_PROTO (auto, ll, ll128, sentinel, direct, barrier, atomic)
 * and AR_WATCHDOG_MS (a positive integer), as NCCL reads NCCL_ALGO and
 * NCCL_PROTO; a value that does not parse, or an impossible pair, fails.
 * The kernels' timers (watchdog budgets, start delays, call timestamps)
 * count the device's constant clock at 100 MHz, the rate MI355X reports as
 * hipDeviceAttributeWallClockRate; a device reporting another rate is
 * refused.
 * Errors: AR_ERR_INVALID (bad sizes, a bad environment override, or a
 * constant clock other than 100 MHz), AR_ERR_STATE (already initialised),
 * AR_ERR_OOM, AR_ERR_HIP.
 */
int ar_init(int n_ranks, size_t max_elems);

/*
 * ar_allreduce -- one AllReduce call, enqueued on `stream` (asynchronous):
 * every rank's input summed element by element, the sum given to every rank
 * ("微秒必争…", section "张量并行与AllReduce"); one-shot = each rank publishes
 * its value, receives and reduces all N in registers (recvReduce) and writes,
 * two-shot = reduce-scatter then all-gather (section "统一原语与API设计" and
 * its table of variants), synchronised by the in-band mechanisms of section
 * "四大核心机制" (see ar_set_options for the choice).
 *   rank_bufs: HOST array of n_ranks DEVICE pointers, rank r's bf16 input [n];
 *              copied by value into the launch, so the host array may be
 *              reused as soon as the call returns (graph-capture safe).
 *   out:       DEVICE bf16 [n_ranks][n]; rank r's copy at out + r*n.  Must not
 *              overlap any input.
 *   n:         elements per rank, 1..max_elems, a multiple of 8.
 *   epoch:     call number within the current step: 1 for the first call
 *              after ar_init / ar_reset / ar_step_end, then previous + 1;
 *              at most 65535.  A call walks its message in rounds through the
 *              staging windows (ar_set_staging); round j of a call uses flag
 *              f + j and buffer (f + j) & 1, f following the previous call's
 *              last flag (for one-round calls the buffer alternates call by
 *              call).
 *   stream:    HIP stream (0 = legacy default stream).
 * All pointers 16-byte aligned.  Inputs must be finite bf16 values; with the
 * sentinel protocol an input equal to 0xFFFF breaks the contract (a receiver
 * would wait for it until the watchdog fires).  Inputs must not be modified
 * until the call has completed on `stream`.  No allocation, memset or host
 * synchronisation happens here.
 * Errors: AR_ERR_NOT_INIT, AR_ERR_INVALID (pointer, size, alignment, aliasing,
 * epoch sequence), AR_ERR_HIP (launch failure).  Device-side failures
 * (watchdog) are reported later through ar_get_status.
 */
int ar_allreduce(const void *const *rank_bufs, void *out, size_t n,
                 uint32_t epoch, hipStream_t stream);

/*
 * ar_allreduce_add_rmsnorm -- one AllReduce call (one-shot, LL protocol)
 * with the operation that follows it in a decode layer fused into the same
 * launch: the residual add and the RMS norm ("vLLM 分布式推理核心" page,
 * section 一: after the AllReduce the compute stream resumes with the norm;
 * the page names the op without defining it, and the weighted RMS form with
 * a residual add is what is computed).  For every rank r and row i of
 * `rows` rows of `hidden` elements (n = rows * hidden):
 *     a       = the AllReduce result (bf16, bit-identical to ar_allreduce)
 *     h[e]    = bf16_rne( f32(a[e]) + f32(residual_r[e]) )
 *     y[e]    = bf16_rne( (f32(h[e]) * s_i) * f32(gamma[e mod hidden]) ),
 *     s_i     = 1 / sqrt( S_i / hidden + eps ),  S_i = binary32 sum of h^2
 *               over row i, in a fixed order that does not depend on the
 *               launch geometry (256-element blocks of 64 x 4 elements).
 *   rank_bufs: HOST array of n_ranks DEVICE pointers, bf16 [n] (as ar_allreduce).
 *   residual:  HOST array of n_ranks DEVICE pointers, rank r's bf16 residual [n].
 *   gamma:     DEVICE bf16 [hidden], the norm weight, shared by all ranks.
 *   eps:       finite, >= 0.
 *   out_h:     DEVICE bf16 [n_ranks][n], the updated residual stream h.
 *   out_y:     DEVICE bf16 [n_ranks][n], the normalised rows y.
 *   rows:      >= 1;  hidden: a multiple of 256, 256..65536;
 *              rows * hidden <= max_elems.
 *   epoch, stream: as ar_allreduce; the call takes the next epoch of the
 *              same sequence, so it mixes freely with ar_allreduce calls.
 * All pointers 16-byte aligned; out_h and out_y must overlap neither each
 * other nor any input, residual or gamma.  The a values themselves are not
 * written out.  h is exact; y is within one bf16 unit in the last place of
 * the exact value (binary32 sum, division, square root and products).  The
 * kernel follows the message: up to 16 KiB per rank the one-shot LL; above
 * it the in-place one-shot (DIRECT), with one workgroup per rank and row
 * for 8 or more rows of at most 8192 elements, else spread over several
 * workgroups per row.  The LL and the spread forms exchange each row's
 * partial sums between workgroups, so their whole grid must be resident at
 * once (the launch stays within half the device's capacity).  ar_set_options
 * may fix LL or DIRECT (one-shot); other protocols and two-shot have no
 * fused form (AR_ERR_INVALID).  All three forms give the same bits.  No
 * allocation, memset or host synchronisation.
 * Errors: as ar_allreduce (AR_ERR_INVALID also for the norm operands).
 */
int ar_allreduce_add_rmsnorm(const void *const *rank_bufs, const void *const *residual,
                             const void *gamma, float eps, void *out_h, void *out_y,
                             size_t rows, size_t hidden, uint32_t epoch, hipStream_t stream);

/*
 * ar_add_rmsnorm -- the same residual add and RMS norm as a kernel of its
 * own, applied to an AllReduce result already in memory (the unfused
 * sequence: ar_allreduce, then this call).
 *   a:         DEVICE bf16 [n_ranks][n], e.g. ar_allreduce's out.
 *   residual, gamma, eps, out_h, out_y, rows, hidden: as ar_allreduce_add_rmsnorm;
 *              out_h and out_y must not overlap a either.
 * Needs an initialised context (for n_ranks and max_elems); uses no epoch.
 * Same arithmetic and summation order as the fused call, so for the same a
 * both give identical h and y.  One workgroup of 1024 threads per (rank, row).
 * Errors: AR_ERR_NOT_INIT, AR_ERR_INVALID, AR_ERR_HIP.
 */
int ar_add_rmsnorm(const void *a, const void *const *residual, const void *gamma, float eps,
                   void *out_h, void *out_y, size_t rows, size_t hidden, hipStream_t stream);

/*
 * ar_allreduce_f32_debug -- the same call, but writes the binary32
 * accumulators (before the bf16 rounding) to out_f32, DEVICE float
 * [n_ranks][n]: the register sums of recvReduce ("微秒必争…", section
 * "统一原语与API设计") made visible, for checking the fold itself.  Same
 * contract otherwise (device scope always); advances the epoch sequence
 * like ar_allreduce.
 */
int ar_allreduce_f32_debug(const void *const *rank_bufs, float *out_f32,
                           size_t n, uint32_t epoch, hipStream_t stream);

/*
 * ar_allreduce_noalloc -- the same AllReduce for callers that cannot
 * allocate: code under hipGraph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  Neither this call nor any set-up allocates, and it
 * needs no ar_init: it runs the one-shot sentinel protocol with its inboxes
 * in a static device array of 4 MiB per device (held until the process
 * ends), whose address it takes with hipGetSymbolAddress on its first call
 * on each device.  Sentinel validity is in-band and every consumed inbox
 * slot is re-armed within the call, so no flag sequence or step end is
 * needed; the window per (receiver, sender) pair and buffer is
 * 4 MiB / (2 n_ranks^2), at most 64 KiB, walked in rounds for larger
 * messages.  Device-scope coherence (no placement probe runs).
 *   rank_bufs, out, stream: as ar_allreduce; inputs must not hold 0xFFFF.
 *   n:         elements per rank, a multiple of 8, with all n_ranks output
 *              copies within 2^31 bytes (AR_ERR_INVALID beyond that); n == 0
 *              re-arms this device's inboxes (needed only after a call that a
 *              watchdog ended) and launches nothing else.
 *   n_ranks:   1..16.
 * The first call on a device also enqueues the arming of its inboxes (a
 * fill kernel, capture-safe; inside a capture it is captured, and the next
 * call outside one arms again).  Every call on a device shares its array:
 * calls that overlap on one device (different streams, no ordering) race.
 * Single host thread.  A watchdog failure is recorded in the status record
 * that ar_get_status reads (when a context exists); that call's outputs
 * are undefined until a call with n == 0.
 * Errors: AR_ERR_INVALID (sizes, pointers, alignment, aliasing), AR_ERR_HIP.
 */
int ar_allreduce_noalloc(const void *const *rank_bufs, void *out, size_t n, int n_ranks,
                         hipStream_t stream);

/*
 * ar_destroy -- free all staging (the counterpart of ar_init; the pages'
 * library is a drop-in behind the collective's interface, "SiFAR" page,
 * section "实际部署考量").  The caller must have synchronised every stream
 * that used the library.  AR_ERR_NOT_INIT if there is no context.
 */
int ar_destroy(void);

/*
 * ar_set_options -- choose the algorithm and protocol for later calls.
 * AUTO picks by message size S = 2n bytes per rank, as measured on MI355X
 * (the pages' table of variants in section "统一原语与API设计" puts the
 * one-shot/two-shot crossover at 64 KB on NVLink; in-place one-shot reads
 * stay ahead much longer here): S < 1 MiB -> one-shot DIRECT; otherwise
 * two-shot DIRECT.  (The fused ar_allreduce_add_rmsnorm uses its LL form
 * up to S = 16 KiB under AUTO.)  With a protocol fixed and
 * the algorithm AUTO, one-shot is used up to that protocol's crossover
 * (sentinel 64 KiB, LL128 128 KiB, DIRECT and barrier just below 1 MiB);
 * LL is always one-shot and the atomic lines always two-shot.
 * AR_ERR_INVALID for an unknown value or an impossible pair.
 */
int ar_set_options(int algo, int proto);

/*
 * ar_set_launch -- tuning (the per-optimisation controls of a drop-in
 * collective, "SiFAR" page, section "实际部署考量"): workgroups per rank
 * (0 = automatic) and threads per workgroup (64, 128 or 256; 0 = automatic).  The LL kernel always
 * uses one wave per rank (64 x the next power of two >= N threads), the
 * sentinel kernels 512 threads and the LL128 kernels 256: their waves share
 * the peers of a tile.  The
 * workgroups per rank are capped at each call so that the whole grid is
 * resident at once (every poll then has a running producer).
 * AR_ERR_INVALID for unsupported values.
 */
int ar_set_launch(int wgs_per_rank, int threads);

/*
 * ar_set_scope -- coherence scope of the staging buffers and flag words
 * (enum ar_scope; default AR_SCOPE_AUTO).  XCD-local scope serves every
 * exchange from the L2 of the XCD its writer and reader share: stores at
 * workgroup scope and streaming workgroup-scope polls instead of
 * device-scope accesses.  Each workgroup of such a launch takes the low
 * bits of its part index from the XCD it runs on, which keeps the exchanges
 * XCD-local whichever XCD the round-robin dispatch starts from; ar_init
 * checks the round-robin order with probe launches (ar_query key 9) and
 * leaves the scope off if it does not hold.  AR_SCOPE_CROSS_XCD instead
 * places the ranks across the XCDs (rank r on XCD r mod 8) with device-scope
 * accesses, so that the ranks' exchanges cross the XCDs' L2s as a real
 * tensor-parallel exchange crosses the fabric between GPUs ("微秒必争…",
 * section "张量并行与AllReduce": the communication after each layer that the
 * method speeds up).  The fp32 debug path always uses device scope.  Returns
 * AR_ERR_INVALID for other values.
 */
int ar_set_scope(int scope);

/*
 * ar_set_staging -- size of the staging window the staged protocols walk
 * their rounds through (the double buffering of "微秒必争…", section
 * "四大核心机制", item 3: a message larger than one exchange goes in rounds
 * through buffers 0 and 1, and receiving a peer's round k permits
 * overwriting the buffer of round k-1).  ar_init allocates, per rank and
 * buffer, min(what the largest message needs, 1 MiB) for LL and LL128, and
 * per (receiver, sender) inbox and buffer min(need, 256 KiB) for the
 * sentinel protocol; this call limits the window actually used to
 * window_bytes (a multiple of 1024, at least 4096; 0 = the whole
 * allocation).  Each call then runs as many parts as one round of each fits
 * the window (1 KiB per part and round; LL128: 1 KiB per line group of a
 * batch) and as many rounds as the message needs; round j of a call uses
 * buffer (f + j) & 1 with flag f + j, where f is the call's first flag.
 * Takes effect for the following calls.  Errors: AR_ERR_NOT_INIT,
 * AR_ERR_INVALID.
 */
int ar_set_staging(size_t window_bytes);

/*
 * ar_set_watchdog -- per-poll time budget in microseconds (default 200000,
 * or AR_WATCHDOG_MS at ar_init).  It bounds the waits the flag protocols
 * introduce: a sentinel receiver whose data never leaves the sentinel
 * pattern would otherwise wait forever ("微秒必争…", section "四大核心机制",
 * item 2).
 * A poll that exceeds it records {6, rank, source, flag} in the device status
 * record and its workgroup stops (in the fused norm's wait for the row's
 * block sums, source is the waiting rank itself); the other workgroups of
 * that call stop polling soon after they see the record.  The record stays until ar_reset;
 * until then outputs of later calls are undefined.  0 restores the default.
 */
int ar_set_watchdog(uint32_t budget_us);

/*
 * ar_step_end -- close a step of calls (typically one emulated decode step of
 * 2 x layers calls: the 160 AllReduces per token of an 80-layer model,
 * "vLLM 分布式推理核心" page, section 一).  Enqueues one tiny kernel on
 * `stream` that advances the device's round sequence by the rounds of the
 * step's calls and its call count by their number, so that the flags of a
 * captured hipGraph's replays never repeat, and clears the arrival words of
 * the in-place kinds (whose values are positions within the step); resets
 * the host epoch counter to 0.  Buffer parity follows the global round
 * number, so a step may hold any number of calls.  When the round sequence passes 0xF0000000 the kernel
 * clears every flag word and restarts it at 0.  A step holds at most 2^27
 * rounds (ar_allreduce refuses a call beyond that).
 * Errors: AR_ERR_NOT_INIT, AR_ERR_HIP.
 */
int ar_step_end(hipStream_t stream);

/*
 * ar_set_sequence -- test hook for the flag sequence that tags every round
 * (the double buffering of "微秒必争…", section "四大核心机制", item 3, needs
 * a flag unique to each round): sets the device round sequence to `seq`
 * (<= 0xF0000000) with a kernel on `stream`, so that a test can run steps
 * across the sequence's restart.  Only between steps (AR_ERR_STATE after a
 * call of an open step).  Errors: AR_ERR_NOT_INIT, AR_ERR_STATE,
 * AR_ERR_INVALID, AR_ERR_HIP.
 */
int ar_set_sequence(uint32_t seq, hipStream_t stream);

/*
 * ar_set_delays -- test hook: per (call, rank) start delays, so that ranks
 * arrive at a call at different times as real GPUs do (the slowest one
 * sets the pace: the small-message essay, section 4.2; "SiFAR" page,
 * section "技术三").  dev_ns is a
 * DEVICE uint32 table [calls][n_ranks] of nanoseconds; call with flag f uses
 * row (f - 1) mod calls.  Every workgroup of rank r spins on the constant
 * 100 MHz clock for that long before its first step.  NULL disables.  The
 * table must stay alive while calls use it.
 */
int ar_set_delays(const uint32_t *dev_ns, size_t calls);

/*
 * ar_set_timestamps -- measurement hook (time completion at the consumer,
 * not at the asynchronous return: the small-message essay, section 6.2):
 * DEVICE uint64 table [slots][records_per_slot][4], zeroed by the caller.
 * For the call numbered c (calls counted from 1 since ar_init / ar_reset,
 * across steps) the kernels write into slot (c - 1) mod slots, in ticks of
 * the constant 100 MHz clock, with plain stores (no atomics, waits or
 * barriers):
 *   phases == 0: wave 0 of every workgroup writes its start time into field
 *                0 of record w = the workgroup's position in dispatch order,
 *                in the prologue (a store issued at a workgroup's end would
 *                itself lengthen the call); the period of call k is then
 *                start(k+1) - start(k), start = the earliest record;
 *   phases != 0: every wave writes at its end record w = workgroup position
 *                x waves per workgroup + wave = {start, first synchronisation
 *                satisfied, last data store issued, end} (each mark is one
 *                more read of the clock, and the late stores lengthen the
 *                call).
 * Records with w >= records_per_slot are not written.  NULL disables (the
 * default).  records_per_slot should be at least the launch's workgroup
 * count (ar_query key 4), or its wave count with phases (keys 4 and 5).
 * Errors: AR_ERR_NOT_INIT, AR_ERR_INVALID (zero sizes, or a table above
 * 2^40 records).
 */
int ar_set_timestamps(uint64_t *dev_ts, size_t slots, size_t records_per_slot, int phases);

/*
 * ar_get_status -- copy the device status record {code, rank, source, call}
 * into out[4] (synchronises the device first).  code is 0 or 6 (a watchdog
 * fired -- the deadlock a lost sentinel would cause, "微秒必争…", section
 * "四大核心机制", item 2 -- with the rank that gave up, the source it waited
 * for and the call number, counted from 1 since ar_init / ar_reset).
 * Returns AR_ERR_TIMEOUT if a watchdog fired, else AR_OK.
 */
int ar_get_status(uint32_t out[4]);

/*
 * ar_reset -- recovery (the resetRange() of section "统一原语与API设计"):
 * enqueues kernels on `stream` that zero every flag word, re-arm every
 * sentinel buffer, clear the status record and restart the flag sequence;
 * resets the host epoch counter.  Graph-capture safe (no memset nodes).
 */
int ar_reset(hipStream_t stream);

/* ar_strerror -- static description of a status code (the library reports
 * rather than aborts, as a drop-in collective must: "SiFAR" page, section
 * "实际部署考量"). */
const char *ar_strerror(int status);

/* ar_last_hip_error -- the hipError_t behind the last AR_ERR_HIP (same
 * reason as ar_strerror). */
int ar_last_hip_error(void);

/*
 * ar_query -- introspection for tests and benchmarks (what NCCL_DEBUG=INFO
 * reports per collective -- chosen algorithm, protocol, geometry -- the
 * small-message essay, section 4.4).  key:
 *   0 n_ranks, 1 max_elems, 2 algorithm a call of n elements would use,
 *   3 its protocol, 4 workgroups it would launch, 5 threads per workgroup,
 *   6 resident-workgroup capacity of the device for that kernel, 7 the host
 *   epoch counter, 8 1 if a call of n elements would use XCD-local scope
 *   (else 0), 9 1 if ar_init verified the round-robin XCD placement,
 *   10 the constant-clock rate in kHz, 11 the device's compute-unit count.
 * Returns the value, or a negative status.
 */
long long ar_query(int key, size_t n);
/*   (continued) 16 1 if a call of n elements would place rank r on XCD r mod 8
 *   (grid (1, N, parts)), 0 if part p of every rank on XCD p mod 8,
 *   12 rounds (flags) a call of n elements would take, 13 rounds of
 *   the open step so far, 14 the device round sequence (n == 0) or call count
 *   (n != 0), read after a device synchronisation, 15 the staging window
 *   (bytes per rank or inbox pair and buffer) the protocol of a call of n
 *   elements walks (0 for protocols without staging). */

#ifdef __cplusplus
}
#endif
#endif /* TPDC_AR_H */
