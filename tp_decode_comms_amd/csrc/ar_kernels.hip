// ar_kernels.hip -- gfx950 kernels of the barrier-free fixed-order AllReduce.
//
// One launch = one AllReduce call for all N emulated ranks; each workgroup
// covers one part of one rank's work (mapping in begin()).  The hardware
// dispatches workgroups to the 8 XCDs round-robin by index, and the host
// makes `parts` a multiple of 8, so part p of every rank runs on XCD p % 8:
// all traffic of one part (mailboxes, inboxes, lines, arrival and completion
// flags) stays inside one XCD's L2.  With device-scope accesses correctness
// does not depend on that placement, only latency does; the XCD-local scope
// derives the part from the XCD each workgroup runs on, so its exchanges are
// XCD-local by construction.  Workgroups of one part index depend only on each other and are
// dispatched together, and the host never launches more workgroups than the
// device holds at once, so every poll has a producer that runs.
//
// Algorithms ("Every Microsecond Counts" write-up, page "微秒必争…", section
// "统一原语与API设计" and its table of variants):
//   one-shot: read local value, publish, receive-and-reduce all N, write;
//   two-shot: reduce-scatter (rank q reduces slice q) then all-gather.
// Protocols (same page, section "四大核心机制"): LL units, sentinel inboxes,
// parity double buffering, LL128-style lines; plus DIRECT, in which a rank
// announces its arrival with a counter and peers read its input in place
// (one-shot) or receive the reduced slices straight into their outputs
// (two-shot), completion announced by per-workgroup flags.
//
// Summation order is the global rank order 0..N-1 for every element on
// every rank and in both algorithms, so all variants give identical bits.
//
// Latency notes (measured on MI355X): a line written by one XCD with the
// device-scope policy becomes readable by another XCD about 1 us later, by
// the same XCD about 0.5-0.9 us later; a wave's loads cannot be consumed
// before its earlier stores are acknowledged (one in-order counter for
// both).  Polls therefore keep two batches of loads in flight, start only
// after the wave's own publish is acknowledged (a poll issued earlier mostly
// returns stale data and costs a second round trip), and flag words are tiny
// and read by few lanes.
#include "ar_proto.h"
#include "ar_kernels.h"
#include "norm_math.h"

namespace ar {

// The control block (CTL_WORDS words: the sequence words, the status record,
// the arrival and barrier words; layout in ar_proto.h).  A file-scope device
// array rather than an allocation: its address is a link-time constant, so
// a kernel's load of the sequence words does not wait for the launch record
// to arrive first -- it goes out with the record's own loads, one memory
// round trip earlier (the arrival flags of the in-place kernels depend on
// it).  One block per device; the host takes its address with
// hipGetSymbolAddress (control_block()) and the launch record carries it for
// every other use.
__device__ __align__(256) uint32_t ar_control[CTL_WORDS];

hipError_t control_block(uint32_t **p)
{
    return hipGetSymbolAddress((void **)p, HIP_SYMBOL(ar_control));
}

// ------------------------------------------------------------------ common
// flag: the flag of the call's first round (round j uses flag + j); call:
// the call's number since the last reset (start delays, measurement slots,
// status records); par: buffer parity of the first round (flag & 1).
struct Ctx0 {
    uint32_t rank, part, flag, call, par;
    uint32_t seq, calls;            // the sequence words, fetched in the prologue
    bool delay;                     // a start-delay table is set
    bool stamp;                     // a timestamp table of start records is set
    bool phases;                    // a timestamp table with phase records is set
    uint64_t t0, t_sync, t_data;
};

// The workgroup's position in dispatch order, x + X (y + N z) on the grid
// (X, N, parts / X) described at begin().
__device__ __forceinline__ uint32_t linear_id(const Launch &a)
{
    return ((blockIdx.z * a.n_ranks + blockIdx.y) << a.xshift) + blockIdx.x;
}

// The two sequence words {round sequence, call count} of the step.  Only the
// step-end kernel and the host's re-arm kernels write them, always in an
// earlier launch; the launch boundary makes that write visible, and no launch
// writes them while an AllReduce kernel runs, so they are read as constant
// memory: one scalar load, served by the scalar cache a CU's waves share
// (every wave of the launch reads them; 8 x 16 KiB LL: 2.63 -> 2.58 us per
// call against a vector load), from the control block's fixed address, in
// the prologue's load round (begin()).
__device__ __forceinline__ u32x2 seq_words()
{
    typedef const __attribute__((address_space(4))) u32x2 const_u32x2;
    return *((const_u32x2 *)ar_control + CTL_SEQ / 2);
}

__device__ __forceinline__ void stamp_start(const Launch &a, const Ctx0 &c);

// The call's flag, number and first buffer parity from the sequence words.
__device__ __forceinline__ void load_seq(const Launch &a, Ctx0 &c)
{
    c.flag = c.seq + a.rbase + 1u;
    c.call = c.calls + a.epoch;
    c.par = c.flag & 1u;
    stamp_start(a, c);
}

__device__ __forceinline__ void start_delay(const Launch &a, const Ctx0 &c)
{
    if (!c.delay)
        return;
    __amdgpu_buffer_rsrc_t d = rsrc(a.delays, a.delay_rows * a.n_ranks * 4u);
    uint32_t row = (c.call - 1u) % a.delay_rows;
    uint32_t ns = ld4<CP_PLAIN>(d, (row * a.n_ranks + c.rank) * 4u);
    uint64_t ticks = ns / 10u;
    if (ticks > 1000000u)                 // at most 10 ms per call
        ticks = 1000000u;
    while (clock100() - c.t0 < ticks)
        __builtin_amdgcn_s_sleep(1);
}

// Phase marks (only with a timestamp table asking for them): `mark` records
// the clock, `mark_once` only the first time.  Each read of the constant
// clock is a scalar-memory instruction whose result the next LDS or scalar
// wait also waits for, so marks on the critical path lengthen the call
// (8 x 16 KiB LL: +0.37 us per call with both marks); a table without them
// records only the start (read anyway) and the end.
__device__ __forceinline__ void mark(const Ctx0 &c, uint64_t &t)
{
    if (c.phases)
        t = clock100();
}
__device__ __forceinline__ void mark_once(const Ctx0 &c, uint64_t &t)
{
    if (c.phases && t == 0u)
        t = clock100();
}

// Measurement records (only with a timestamp table).  Without phases, lane 0
// of each workgroup's wave 0 writes its start time into record [slot][w]
// (w: the workgroup's position in dispatch order, slot: (call - 1) mod
// slots) as soon as the call number is known, with one plain store: no
// atomic, wait or barrier.  The store completes long before the kernel ends,
// so the call runs as it does without the table (a store issued as a
// workgroup's last instruction measured 0.2 us longer per 16 KiB call:
// the launch completes only once every store has been acknowledged).  Call
// k's period is start(k+1) - start(k).  With phases every wave writes its
// whole record {start, first synchronisation satisfied, last data store
// issued, end} at its end instead, which lengthens the call.
__device__ __forceinline__ void stamp_start(const Launch &a, const Ctx0 &c)
{
    if (!c.stamp || threadIdx.x != 0u)
        return;
    const uint32_t w = linear_id(a);
    if (w >= a.ts_stride)
        return;
    const uint32_t slot = (c.call - 1u) % a.ts_slots;
    a.ts[((size_t)slot * a.ts_stride + w) * TS_FIELDS] = c.t0;
}

__device__ __forceinline__ void finish(const Launch &a, const Ctx0 &c)
{
    if (!c.phases || (threadIdx.x & 63u) != 0u)
        return;
    const uint64_t t1 = clock100();
    const uint32_t w = linear_id(a) * (blockDim.x >> 6) + (threadIdx.x >> 6);
    if (w >= a.ts_stride)
        return;
    const uint32_t slot = (c.call - 1u) % a.ts_slots;
    uint64_t *p = a.ts + ((size_t)slot * a.ts_stride + w) * TS_FIELDS;
    p[0] = c.t0;
    p[1] = c.t_sync;
    p[2] = c.t_data;
    p[3] = t1;
}

// HOOKS: which measurement and test hooks the kernel is built with -- 0
// none, 1 the start records only (a timestamp table without phases), 2 all
// (start delays, start records or per-wave phase records).  A kernel built
// without a hook carries none of its code: even a hook disabled at run time
// cost (8 x 16 KiB LL 2.43 -> 2.38 us, 8 x 64 KiB LL 3.86 -> 3.40,
// 8 x 16 KiB in-place one-shot 2.35 -> 2.26 once removed).  The host picks
// the twin from the tables that are set.
template <bool LOCAL, int HOOKS>
__device__ __forceinline__ void begin(const Launch &a, Ctx0 &c)
{
    // The start time is read only by the hook twins (start delays, records):
    // a clock read is a scalar-memory instruction, and the register it
    // writes had to be waited for before the prologue could reuse it
    // (8 x 4 MiB two-shot 12.80 -> 12.65 us, 8 x 16 KiB in-place one-shot
    // 2.18 -> 2.13, same box, once gone from the hook-free kernels).
    c.t0 = HOOKS != 0 ? clock100() : 0u;
    c.t_sync = 0u;
    c.t_data = 0u;
    // The grid is (X, N, parts / X) with X = 2^xshift consecutive parts of
    // one rank along x (X = 8 when parts is a multiple of 8, else 1): the
    // rank is blockIdx.y and the part (blockIdx.z << xshift) + blockIdx.x.
    // Workgroups are dispatched in linear order x + X (y + N z), so blocks
    // of X*N consecutive workgroups hold parts zX .. zX+X-1 of every rank:
    // with X = 8 part p lands on XCD p % 8, every workgroup's peers (same
    // part, other ranks) sit in its own block, and parts 0..7 of every rank
    // (arrival writers, completion waiters) in the first, so progress never
    // needs more than one block resident.  Rank and part come from the
    // workgroup id itself, so nothing in the prologue waits for a load
    // before the rank's own pointers can be fetched.
    c.rank = blockIdx.y;
    // The XCD-local scope takes the low three part bits from the XCD the
    // workgroup actually runs on.  Dispatch is round-robin from some XCD o
    // (o = 0 normally; a profiler can shift it), so within each group of 8
    // consecutive workgroups of one rank the XCDs are a rotation of 0..7:
    // the mapping stays one-to-one and part p always runs on XCD p % 8,
    // whatever o is.  (ar_init checks the round-robin order, for this grid
    // shape too, before it enables this scope.)
    const uint32_t lo = LOCAL ? xcc_id() : blockIdx.x;
    // The launch record lives in memory that is read cold at every launch:
    // each round of dependent loads from it costs a memory round trip before
    // the first data load can go out.  Handing the fields every kernel uses
    // to an empty asm statement makes the compiler issue all of them at once
    // (the rank's own input pointer included, whose address depends only on
    // blockIdx.y) behind a single wait.
    // (blockDim.x is read from the launch's hidden arguments, so it is one
    // of them; so is the watchdog budget, which the first poll loop reads:
    // loaded there, its scalar load was waited for with the LDS accesses
    // after the first poll -- 8 x 16 KiB LL 2.37-2.38 -> 2.34 us, 8 x 512
    // KiB LL128 two-shot 4.37 -> 4.31, same box.)
    // (The sequence words come with them: their address is a constant.)
    const u32x2 sq = seq_words();
    if constexpr (HOOKS == 2)
        asm volatile("" ::"s"(a.in[c.rank]), "s"(a.out), "s"(a.ctl), "s"(a.n), "s"(a.n_ranks),
                     "s"(a.epoch), "s"(a.rbase), "s"(a.parts), "s"(a.slice), "s"(a.xshift),
                     "s"(a.delays), "s"(a.ts), "s"(a.ts_slots), "s"(a.ts_stride),
                     "s"(a.ts_phases), "s"(sq), "s"(blockDim.x), "s"(a.watchdog_ticks));
    else if constexpr (HOOKS == 1)
        asm volatile("" ::"s"(a.in[c.rank]), "s"(a.out), "s"(a.ctl), "s"(a.n), "s"(a.n_ranks),
                     "s"(a.epoch), "s"(a.rbase), "s"(a.parts), "s"(a.slice), "s"(a.xshift),
                     "s"(a.ts), "s"(a.ts_slots), "s"(a.ts_stride), "s"(sq), "s"(blockDim.x), "s"(a.watchdog_ticks));
    else
        asm volatile("" ::"s"(a.in[c.rank]), "s"(a.out), "s"(a.ctl), "s"(a.n), "s"(a.n_ranks),
                     "s"(a.epoch), "s"(a.rbase), "s"(a.parts), "s"(a.slice), "s"(a.xshift),
                     "s"(sq), "s"(blockDim.x), "s"(a.watchdog_ticks));
    c.seq = sq.x;
    c.calls = sq.y;
    c.part = (blockIdx.z << a.xshift) + lo;
    // after the fields' loads are issued (computed earlier, the test of a.ts
    // made the compiler wait for it before issuing the others)
    c.delay = HOOKS == 2 && a.delays != nullptr;
    c.stamp = HOOKS == 1 ? a.ts != nullptr : (HOOKS == 2 && a.ts != nullptr && a.ts_phases == 0u);
    c.phases = HOOKS == 2 && a.ts != nullptr && a.ts_phases != 0u;
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t in_rsrc(const Launch &a, uint32_t r)
{
    return rsrc(a.in[r], a.n * 2u);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t out_rsrc(const Launch &a, uint32_t r, bool f32)
{
    const uint32_t esz = f32 ? 4u : 2u;
    return rsrc((char *)a.out + (size_t)r * a.n * esz, a.n * esz);
}

// All N output copies under one descriptor (the host bounds N*n*4 < 2^32);
// copy r starts at byte r*n*esz.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t out_all(const Launch &a, bool f32)
{
    const uint32_t esz = f32 ? 4u : 2u;
    return rsrc(a.out, a.n_ranks * a.n * esz);
}

// 8 accumulated elements -> out[rank][elem..elem+8)
template <bool F32, int CP = CP_PLAIN>
__device__ __forceinline__ void store8(__amdgpu_buffer_rsrc_t o, uint32_t elem, const Acc8 &acc)
{
    if constexpr (F32) {
        u32x4 lo, hi;
        lo.x = __float_as_uint(acc.v[0]); lo.y = __float_as_uint(acc.v[1]);
        lo.z = __float_as_uint(acc.v[2]); lo.w = __float_as_uint(acc.v[3]);
        hi.x = __float_as_uint(acc.v[4]); hi.y = __float_as_uint(acc.v[5]);
        hi.z = __float_as_uint(acc.v[6]); hi.w = __float_as_uint(acc.v[7]);
        st16<CP>(lo, o, elem * 4u);
        st16<CP>(hi, o, elem * 4u + 16u);
    } else {
        st16<CP>(acc.bf16(), o, elem * 2u);
    }
}

// 4 accumulated elements (in v[0..3]) -> out[rank][elem..elem+4)
template <bool F32, int CP = CP_PLAIN>
__device__ __forceinline__ void store4(__amdgpu_buffer_rsrc_t o, uint32_t elem, const float *v)
{
    if constexpr (F32) {
        u32x4 lo;
        lo.x = __float_as_uint(v[0]); lo.y = __float_as_uint(v[1]);
        lo.z = __float_as_uint(v[2]); lo.w = __float_as_uint(v[3]);
        st16<CP>(lo, o, elem * 4u);
    } else {
        u32x2 w; w.x = pack_bf16(v[0], v[1]); w.y = pack_bf16(v[2], v[3]);
        st8<CP>(w, o, elem * 2u);
    }
}

// 2 accumulated elements (in v[0..1]) -> out[rank][elem..elem+2)
template <bool F32, int CP = CP_PLAIN>
__device__ __forceinline__ void store2(__amdgpu_buffer_rsrc_t o, uint32_t elem, const float *v)
{
    if constexpr (F32) {
        u32x2 w; w.x = __float_as_uint(v[0]); w.y = __float_as_uint(v[1]);
        st8<CP>(w, o, elem * 4u);
    } else {
        st4<CP>(pack_bf16(v[0], v[1]), o, elem * 2u);
    }
}

// Output-store cache policies.  Outputs are never read inside the launch,
// and every line a launch leaves dirty in an L2 is written back at the
// launch boundary before the next launch may start.  A non-temporal store
// (nt, no scope bit) streams its line out without that write-back and
// without waiting for memory on the way: 8 x 512 KiB in-place one-shot
// 4.31 -> 4.10 us per call, and the line-protocol kernels below gain more;
// 8 x 16 KiB one-shot LL is unchanged (2.43), and there it stays plain.
// Streaming device-scope stores (nt with sc1, written through to memory
// inside the launch) cost: 8 x 16 KiB LL 2.44 -> 2.99 us, 8 x 16 KiB
// in-place one-shot 2.35 -> 2.46.
constexpr int LL_OUT = CP_PLAIN;
constexpr int D1_OUT = CP_NT;
constexpr int SENT_OUT = CP_NT;         // sentinel kernels (16 x 57344 two-shot 5.60 -> 5.49 us)
// The fused-norm kernels store h and y non-temporal too (CP_NT at each
// store): 8 x 512 KiB fused AllReduce + norm 6.64 -> 5.90 us per call.

// ============================================================ arrivals
// Rank s announces "my input for this call is final" by storing the flag of
// the call's first round f (sequence word + the step's earlier rounds + 1)
// into its arrival word as soon as the prologue's load round has returned.
// Flags grow monotonically between restarts, so a reader needs word >= f
// (wrap-safe compare).  The word is replicated per XCD: parts x < 8 of rank
// s write copy x, and part p reads copy p % 8, which the same-XCD part of
// every peer wrote.  The N words of one copy share one 128-byte line, so a
// reader polls a single line (polls of lines written during the launch are
// costly for the L2).  Only kinds that read peers' data in place (DIRECT,
// the in-place fused norms, the LL128 two-shot's reduce-scatter) use
// arrivals.  (Raising them with atomics at the first instruction instead,
// before the sequence word arrives, measured slower: the atomics complete
// later than a store is seen by a poll in the XCD's L2.)
__device__ __forceinline__ uint32_t arrive_off(uint32_t copy, uint32_t rank)
{
    return (CTL_ARRIVE + 32u * copy + rank) * 4u;
}

// A call's arrival value: its first round's position in the step (the rounds
// of the step's earlier calls, + 1).  It needs no sequence word; the step end
// clears the arrival words, so within a step the values only grow.
__device__ __forceinline__ uint32_t arrival_value(const Launch &a) { return a.rbase + 1u; }

template <bool LOCAL>
__device__ __forceinline__ void raise_arrival(const Launch &a, const Ctx0 &c)
{
    if (c.part < (uint32_t)XCDS && threadIdx.x == 0)
        st4<Pol<LOCAL>::ST>(arrival_value(a), rsrc(a.ctl, CTL_WORDS * 4u), arrive_off(c.part, c.rank));
}

// The arrival raised at a launch's first instruction, for kernels that take
// the value as a leading argument (the build preloads the first kernel
// argument into a register): with the XCD-local scope the writers (parts
// 0..7) are block 0, their copy is their XCD's and the control block's
// address is a link-time constant, so the store waits for no load.  With
// start delays (HOOKS 2) the rank arrives after its delay instead.  Same-box
// A/B, 160-call graphs, against the sequence-based value raised after the
// prologue: 8 x 4 MiB two-shot 13.18-13.29 -> 13.00-13.17 us (in three
// fresh-allocation passes per process 11.95-12.11 -> 11.88-11.99 on the
// faster allocations), 8 x 512 KiB LL128 two-shot (arrival value only)
// 4.46-4.49 -> 4.35-4.37; the 16 KiB calls unchanged.
template <bool LOCAL, int HOOKS>
__device__ __forceinline__ void raise_arrival_first(uint32_t arr)
{
    if constexpr (LOCAL && HOOKS != 2)
        if (blockIdx.z == 0u && threadIdx.x == 0u)
            st4<Pol<true>::ST>(arr, rsrc(ar_control, CTL_WORDS * 4u), arrive_off(xcc_id(), blockIdx.y));
}
template <bool LOCAL, int HOOKS>
__device__ __forceinline__ void raise_arrival_late(const Launch &a, const Ctx0 &c)
{
    if constexpr (!LOCAL || HOOKS == 2)
        raise_arrival<LOCAL>(a, c);
}

// The first arrival poll of an XCD-local workgroup, issued at the launch's
// first instruction: the control block's address is a link-time constant
// and the copy the workgroup reads is the one of the XCD it runs on, so the
// poll needs nothing from the launch record and travels with its loads.
// Lane l reads rank (l mod 16)'s word; wait_arrivals checks it first.
__device__ __forceinline__ uint32_t early_arrival_poll()
{
    return ld4<Pol<true>::LD>(rsrc(ar_control, CTL_WORDS * 4u),
                              arrive_off(xcc_id(), (threadIdx.x & 63u) & (MAX_RANKS - 1u)));
}

// Every wave waits (two polls in flight) until all N arrival words of its
// XCD's copy reach the call's flag.  Lanes 0..N-1 each watch one word.
// `first`, if given, is the value of an early poll of the same word.
template <bool LOCAL>
__device__ __forceinline__ bool wait_arrivals(const Launch &a, const Ctx0 &c, const Ctl &ctl,
                                              const uint32_t *first = nullptr)
{
    const uint32_t tgt = arrival_value(a);
    const uint32_t lane = threadIdx.x & 63u;
    bool need = lane < a.n_ranks;
    const uint32_t off = arrive_off(c.part % (uint32_t)XCDS, lane & (MAX_RANKS - 1u));
    const __amdgpu_buffer_rsrc_t r = rsrc(a.ctl, CTL_WORDS * 4u);
    Watch w;
    w.begin(a.watchdog_ticks);
    uint32_t v0 = first != nullptr ? *first : (need ? ld4<Pol<LOCAL>::LD>(r, off) : tgt), v1;
    while (true) {
        compiler_fence();
        v1 = need ? ld4<Pol<LOCAL>::LD>(r, off) : tgt;
        if (need && (int32_t)(v0 - tgt) >= 0)
            need = false;
        if (!wave_any(need))
            return true;
        if (w.expired(ctl, c.rank, lane, c.call))
            return false;
        compiler_fence();
        v0 = need ? ld4<Pol<LOCAL>::LD>(r, off) : tgt;
        if (need && (int32_t)(v1 - tgt) >= 0)
            need = false;
        if (!wave_any(need))
            return true;
    }
}

// Workgroup form: wave 0 polls, the workgroup barrier releases the others
// (a quarter of the polling traffic of 4-wave workgroups).
template <bool LOCAL>
__device__ __forceinline__ bool wait_arrivals_wg(const Launch &a, const Ctx0 &c, const Ctl &ctl,
                                                 const uint32_t *first = nullptr)
{
    __shared__ uint32_t ok;
    if (threadIdx.x < 64u)
        ok = wait_arrivals<LOCAL>(a, c, ctl, first) ? 1u : 0u;
    __syncthreads();
    return ok != 0u;
}

// ============================================================ one-shot LL
// Lane work unit: 4 elements (8 bytes of input) = one 16-byte LL store of
// two units {2 bf16, flag}.  Rank r publishes once into its own mailbox
// [r][buffer]; every rank reads it.  All mailboxes sit in one region
// [rank][2 buffers] x ll_stride under one descriptor.
//
// Fixed-size staging, walked in rounds (the double buffering of the pages'
// item 3): the host caps the parts so that one round of every part -- 64
// chunks x 16 bytes each -- fits a rank's window; round j of part p uses
// window bytes [1024 p, 1024 (p+1)) of buffer (flag + j) & 1 with flag
// flag + j.  A part publishes round j+1 only after it has received round j
// from every peer, and each peer published round j only after receiving
// round j-1: so a receipt of round j is the permit to overwrite round j-1's
// buffer, and no reader ever finds its round's data overwritten.  Every
// round carries its own flag, so the stale round j-2 data a reader may find
// in the buffer never validates.
//
// A workgroup of W >= N waves (one per rank, a power of two) owns 64
// chunks per round.  Wave 0 loads the input and publishes it; once the
// publish is acknowledged, wave s receives peer s and stages its units in
// LDS (the peer tiles, [N][64] x 8 bytes); after a workgroup barrier wave 0
// reduces the N units of each chunk from LDS in global rank order and
// writes the result.  Splitting the peers over the waves matters on this
// chip: a poll of lines written during the launch costs about 60 ns per
// load instruction on top of the L2 latency, so 7 peers polled by one wave
// take ~0.85 us, 2 per wave ~0.55 us and 1 per wave ~0.4 us.  Each wave's
// receive keeps two loads in flight: while one is checked the next is
// already on its way.
//
// `epi(ch, v)` consumes the reduced chunk (4 binary32 sums in v) on wave 0;
// all lanes of wave 0 call it together when the round's chunks are in range.
template <int NMAX, bool LOCAL, bool SPLIT, typename Epi>
__device__ __forceinline__ bool ll_round(const Launch &a, Ctx0 &c, const Ctl &ctl,
                                         __amdgpu_buffer_rsrc_t llr, uint32_t ch, uint32_t C,
                                         uint32_t j, u32x2 x, u32x2 (*stage)[64], uint32_t *failed,
                                         Epi &&epi)
{
    const uint32_t N = a.n_ranks;
    const uint32_t rb = a.ll_stride;
    const uint32_t lane = threadIdx.x & 63u, wave = threadIdx.x >> 6;
    const uint32_t fj = c.flag + j;                 // this round's flag and buffer
    const uint32_t lane_off = (c.part * 64u + lane) * 16u + (fj & 1u) * rb;
    const bool active = ch < C;
    // publish (send/bcast): one copy, read by all N ranks
    if (wave == 0u) {
        if (active)
            st16<Pol<LOCAL>::ST>(ll_pack(x.x, x.y, fj), llr, lane_off + c.rank * 2u * rb);
        stage[c.rank][lane] = x;
        wait_stores();
    }
    // polls start once the publish is acknowledged: an earlier poll mostly
    // returns stale data and costs a second round trip
    __syncthreads();
    // receive (recv): this wave's peer is rank `wave`
    const bool mine = wave < N && wave != c.rank && active;
    bool pend = mine;
    const uint32_t src = lane_off + wave * 2u * rb;
    WatchT<false> w;
    w.begin(a.watchdog_ticks);
    // Poll loads are issued by every lane, those with nothing (left) to
    // receive at OFF_NONE (zeros, no traffic): a load under a branch would
    // make the compiler wait for both polls in flight instead of the older.
    // A unit goes to the LDS tile as soon as it is seen valid, so nothing
    // after the loop reads a poll register.
    u32x4 A0 = ld16<Pol<LOCAL>::LD>(llr, pend ? src : OFF_NONE), A1;
    while (true) {
        compiler_fence();
        A1 = ld16<Pol<LOCAL>::LD>(llr, pend ? src : OFF_NONE);
        if (pend && ll_ready(A0, fj)) {
            pend = false;
            stage[wave][lane] = u32x2{A0.x, A0.z};
        }
        if (!wave_any(pend))
            break;
        if (w.expired(ctl, c.rank, wave, c.call)) {
            *failed = 1u;                           // every wave still meets the barrier
            break;
        }
        compiler_fence();
        A0 = ld16<Pol<LOCAL>::LD>(llr, pend ? src : OFF_NONE);
        if (pend && ll_ready(A1, fj)) {
            pend = false;
            stage[wave][lane] = u32x2{A1.x, A1.z};
        }
        if (!wave_any(pend))
            break;
    }
    mark_once(c, c.t_sync);
    lds_barrier();
    if (*failed)
        return false;
    // recvReduce: global rank order from the staged tile.  Every row of the
    // tile is read (rows of absent ranks hold stale values and are not
    // folded), so the reads go out together instead of one wait per rank.
    // With SPLIT, two waves share the fold, each taking one 32-bit word (two
    // elements) of every chunk: the fold is a chain of dependent additions
    // on one wave, so halving it shortens the tail of the call.
    const uint32_t nfold = SPLIT && (blockDim.x >> 6) >= 2u ? 2u : 1u;
    if (wave < nfold && active) {
        u32x2 t[NMAX];
#pragma unroll
        for (int s = 0; s < NMAX; ++s)
            t[s] = stage[s][lane];
        if (nfold == 2u) {
            float v[2];
#pragma unroll
            for (int s = 0; s < NMAX; ++s) {
                if ((uint32_t)s < N) {
                    const uint32_t w = wave == 0u ? t[s].x : t[s].y;
                    if (s == 0) { v[0] = lo_f(w); v[1] = hi_f(w); }
                    else { v[0] += lo_f(w); v[1] += hi_f(w); }
                }
            }
            epi(ch, wave, v, 2);
        } else {
            Acc4 acc;
#pragma unroll
            for (int s = 0; s < NMAX; ++s) {
                if ((uint32_t)s < N) {
                    if (s == 0) acc.init(t[s].x, t[s].y); else acc.add(t[s].x, t[s].y);
                }
            }
            epi(ch, 0u, acc.v, 4);
        }
    }
    // The poll still in flight when the receive loop ended is waited for
    // only here, after the output is on its way: keeping both poll
    // registers live until now stops the compiler from reusing one of them
    // (and waiting for its load) before the tile is read.
    asm volatile("" ::"v"(A0), "v"(A1));
    lds_barrier();                                  // the tile is reused next round
    return true;
}

template <int NMAX, bool F32, bool LOCAL, int HOOKS>
__global__ __launch_bounds__(1024) void k_oneshot_ll(const Launch a)
{
    __shared__ u32x2 stage[NMAX][64];
    __shared__ uint32_t failed;
    Ctx0 c;
    begin<LOCAL, HOOKS>(a, c);
    asm volatile("" ::"s"(a.ll), "s"(a.ll_stride));  // mailboxes: with the first load round
    const uint32_t C = a.n >> 2;                    // 4-element chunks per rank
    const uint32_t lane = threadIdx.x & 63u, wave = threadIdx.x >> 6;
    const uint32_t step = a.parts * 64u;
    if ((blockDim.x >> 6) < a.n_ranks) {            // the host launches a wave per rank
        if (threadIdx.x == 0)                       // (never otherwise: report, do nothing)
            Ctl{a.ctl}.fail(c.rank, blockDim.x, a.epoch);
        return;
    }
    const __amdgpu_buffer_rsrc_t inr = in_rsrc(a, c.rank);
    const __amdgpu_buffer_rsrc_t o = out_rsrc(a, c.rank, F32);
    if (threadIdx.x == 0)
        failed = 0u;
    // first-round input load is issued together with the sequence load
    uint32_t ch = c.part * 64u + lane;
    u32x2 x = {0u, 0u};
    if (wave == 0u && ch < C)
        x = ld8<CP_PLAIN>(inr, ch * 8u);
    load_seq(a, c);
    const Ctl ctl{a.ctl};
    const __amdgpu_buffer_rsrc_t llr = rsrc(a.ll, a.n_ranks * 2u * a.ll_stride);
    start_delay(a, c);
    // round 0 is straight-line code: its poll loads are issued back to back
    // (inside a loop the compiler's counter bookkeeping would wait before each)
    // the fold's output: all 4 elements of a chunk, or word `w` (2 elements)
    auto out = [&](uint32_t cch, uint32_t w, const float *v, int cnt) {
        if (cnt == 4) store4<F32, LL_OUT>(o, cch * 4u, v);
        else store2<F32, LL_OUT>(o, cch * 4u + 2u * w, v);
    };
    if (!ll_round<NMAX, LOCAL, true>(a, c, ctl, llr, ch, C, 0u, x, stage, &failed, out))
        return;
    // later rounds while the workgroup has chunks left (the same rounds for
    // every peer of the part)
    uint32_t j = 1;
    for (uint32_t base = c.part * 64u + step; base < C; base += step, ++j) {
        ch += step;
        x = (wave == 0u && ch < C) ? ld8<CP_PLAIN>(inr, ch * 8u) : u32x2{0u, 0u};
        if (!ll_round<NMAX, LOCAL, true>(a, c, ctl, llr, ch, C, j, x, stage, &failed, out))
            return;
    }
    mark(c, c.t_data);
    finish(a, c);
}

// ================================================ one-shot LL + add + norm
// The AllReduce with the layer's residual add and RMS norm behind it in the
// same launch (the op that follows the AllReduce in the decode loop,
// "vLLM 分布式推理核心" page, section 一; arithmetic in norm_math.h).  The
// LL rounds run as in k_oneshot_ll; on wave 0 each round's reduced chunk a
// becomes h = bf16(a + res), which is written out, and the round's 256
// elements (one norm block, never split by a row end since the row length
// is a multiple of 256) give one partial sum of squares, published with the
// call's flag as one 8-byte store {sum, flag} at device scope -- the blocks
// of a row are spread over all XCDs.  After its last round wave 0 waits for
// the block sums of each row it holds (two polls in flight), folds them in
// the fixed order, and writes y = bf16(h * r * gamma): h of round 0 from
// registers, of later rounds re-read from its own writes.  Every workgroup
// of a row folds the same sums in the same order, so all of them use the
// same r.  The wait spans all workgroups of a rank, so the whole grid must
// be resident at once (the host keeps it to half the device's capacity).
template <bool LOCAL>
__device__ __forceinline__ bool row_rinv(const NormLaunch &L, const Ctx0 &c, const Ctl &ctl,
                                         __amdgpu_buffer_rsrc_t sr, uint32_t row, uint32_t B,
                                         float *rinv)
{
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t base = c.rank * L.stats_stride + row * B;
    float part = 0.0f;
    for (uint32_t g0 = 0; g0 < B; g0 += 64u) {
        const uint32_t j = g0 + lane;
        bool need = j < B;
        const uint32_t off = (base + (need ? j : 0u)) * 8u;
        float got = 0.0f;
        Watch w;
        w.begin(L.base.watchdog_ticks);
        u32x2 v0 = need ? ld8<CP_DEV>(sr, off) : u32x2{0u, 0u}, v1;
        while (true) {
            compiler_fence();
            v1 = need ? ld8<CP_DEV>(sr, off) : u32x2{0u, 0u};
            if (need && v0.y == c.flag) {
                need = false;
                got = __uint_as_float(v0.x);
            }
            if (!wave_any(need))
                break;
            if (w.expired(ctl, c.rank, c.rank, c.call))
                return false;
            compiler_fence();
            v0 = need ? ld8<CP_DEV>(sr, off) : u32x2{0u, 0u};
            if (need && v1.y == c.flag) {
                need = false;
                got = __uint_as_float(v1.x);
            }
            if (!wave_any(need))
                break;
        }
        part = g0 == 0u ? got : part + got;
    }
    *rinv = rms_inv(wave_sum(part), L.hidden, L.eps);
    return true;
}

template <int NMAX, bool LOCAL, int HOOKS>
__global__ __launch_bounds__(1024) void k_oneshot_ll_norm(const NormLaunch L)
{
    const Launch &a = L.base;
    __shared__ u32x2 stage[NMAX][64];
    __shared__ uint32_t failed;
    Ctx0 c;
    begin<LOCAL, HOOKS>(a, c);
    const uint32_t C = a.n >> 2;                    // 4-element chunks per rank
    const uint32_t lane = threadIdx.x & 63u, wave = threadIdx.x >> 6;
    const uint32_t step = a.parts * 64u;
    const uint32_t rounds = (C + step - 1u) / step;
    if ((blockDim.x >> 6) < a.n_ranks) {            // the host launches a wave per rank
        if (threadIdx.x == 0)
            Ctl{a.ctl}.fail(c.rank, blockDim.x, a.epoch);
        return;
    }
    const uint32_t nb = a.n * 2u;
    const __amdgpu_buffer_rsrc_t inr = in_rsrc(a, c.rank);
    const __amdgpu_buffer_rsrc_t resr = rsrc(L.res[c.rank], nb);
    const __amdgpu_buffer_rsrc_t gr = rsrc(L.gamma, L.hidden * 2u);
    const __amdgpu_buffer_rsrc_t oh = rsrc((char *)a.out + (size_t)c.rank * nb, nb);
    const __amdgpu_buffer_rsrc_t oy = rsrc((char *)L.y + (size_t)c.rank * nb, nb);
    const __amdgpu_buffer_rsrc_t sr = rsrc(L.stats, a.n_ranks * L.stats_stride * 8u);
    if (threadIdx.x == 0)
        failed = 0u;
    uint32_t ch = c.part * 64u + lane;
    u32x2 x = {0u, 0u}, rw = {0u, 0u}, g0 = {0u, 0u};
    if (wave == 0u && ch < C) {
        x = ld8<CP_PLAIN>(inr, ch * 8u);
        rw = ld8<CP_PLAIN>(resr, ch * 8u);
        g0 = ld8<CP_PLAIN>(gr, ((ch * 4u) % L.hidden) * 2u);
    }
    load_seq(a, c);
    const Ctl ctl{a.ctl};
    const __amdgpu_buffer_rsrc_t llr = rsrc(a.ll, a.n_ranks * 2u * a.ll_stride);
    start_delay(a, c);
    u32x2 hk = {0u, 0u};
    auto epi = [&](uint32_t cch, uint32_t, const float *v, int) {   // always 4 elements (no split)
        u32x2 aw;
        aw.x = pack_bf16(v[0], v[1]);
        aw.y = pack_bf16(v[2], v[3]);
        const u32x2 hw = add_round4(aw, rw);
        st8<CP_NT>(hw, oh, cch * 8u);
        hk = hw;
        const float s = wave_sum(sumsq4(hw));
        if (lane == 0u) {
            u32x2 e; e.x = __float_as_uint(s); e.y = c.flag;
            st8<CP_DEV>(e, sr, (c.rank * L.stats_stride + (cch >> 6)) * 8u);
        }
    };
    if (!ll_round<NMAX, LOCAL, false>(a, c, ctl, llr, ch, C, 0u, x, stage, &failed, epi))
        return;
    const u32x2 h0 = hk;
    for (uint32_t it = 1; it < rounds; ++it) {
        ch += step;
        const bool ld = wave == 0u && ch < C;
        x = ld ? ld8<CP_PLAIN>(inr, ch * 8u) : u32x2{0u, 0u};
        rw = ld ? ld8<CP_PLAIN>(resr, ch * 8u) : u32x2{0u, 0u};
        if (!ll_round<NMAX, LOCAL, false>(a, c, ctl, llr, ch, C, it, x, stage, &failed, epi))
            return;
    }
    // normalise (wave 0; the other waves go straight to finish's barrier)
    if (wave == 0u) {
        const uint32_t B = L.hidden / NORM_BLOCK;
        uint32_t have = 0xFFFFFFFFu;
        float r = 0.0f;
        for (uint32_t it = 0; it < rounds; ++it) {
            const uint32_t c0 = c.part * 64u + it * step;      // first chunk (wave-uniform)
            if (c0 >= C)
                break;
            const uint32_t row = (c0 >> 6) / B;
            if (row != have) {
                if (!row_rinv<LOCAL>(L, c, ctl, sr, row, B, &r))
                    break;                                      // watchdog: status recorded
                have = row;
            }
            const uint32_t cc = c0 + lane;
            const u32x2 hw = it == 0u ? h0 : ld8<CP_PLAIN>(oh, cc * 8u);
            const u32x2 gw = it == 0u ? g0 : ld8<CP_PLAIN>(gr, ((cc * 4u) % L.hidden) * 2u);
            st8<CP_NT>(scale4(hw, gw, r), oy, cc * 8u);
        }
    }
    mark(c, c.t_data);
    finish(a, c);
}

// ============================================ one-shot DIRECT + add + norm
// The same fused epilogue on the in-place one-shot, for messages where the
// one-shot DIRECT is the faster AllReduce (batched decode: rows x hidden of
// tens to hundreds of KiB per rank).  Each wave owns a run of consecutive
// 256-element norm blocks: after the arrival flags it reads 8 bytes per lane
// from every rank's input in place, folds them in rank order, and continues
// as the LL-fused kernel does (h, each block's sum of squares published
// with the call's flag, the row's sums folded in the fixed order, y).  The blocks and
// every fold are those of norm_math.h, so h and y equal the LL-fused and
// the stand-alone kernels' bit for bit.  Waves work independently; a wave
// whose wait gives up records it and skips its work but still reaches
// finish().  All workgroups of a rank must be resident at once.
template <int NMAX, bool LOCAL, int HOOKS>
__global__ __launch_bounds__(256) void k_oneshot_direct_norm(const NormLaunch L)
{
    const Launch &a = L.base;
    Ctx0 c;
    begin<LOCAL, HOOKS>(a, c);
    const uint32_t N = a.n_ranks;
    const uint32_t lane = threadIdx.x & 63u, wave = threadIdx.x >> 6;
    const uint32_t blocks = a.n / NORM_BLOCK;                  // per rank
    // wave v of the rank owns a run of R consecutive blocks (R even): runs
    // stay within one row where R divides the row's block count, so a wave
    // waits for one row's sums, and it reduces its blocks in pairs whose
    // loads are in flight together
    const uint32_t W = a.parts * (blockDim.x >> 6);
    const uint32_t v = c.part * (blockDim.x >> 6) + wave;
    const uint32_t R = (((blocks + W - 1u) / W) + 1u) & ~1u;
    const uint32_t bbeg = v * R;
    const uint32_t bend = bbeg + R < blocks ? bbeg + R : blocks;
    const uint32_t nb = a.n * 2u;
    const __amdgpu_buffer_rsrc_t resr = rsrc(L.res[c.rank], nb);
    const __amdgpu_buffer_rsrc_t gr = rsrc(L.gamma, L.hidden * 2u);
    const __amdgpu_buffer_rsrc_t oh = rsrc((char *)a.out + (size_t)c.rank * nb, nb);
    const __amdgpu_buffer_rsrc_t oy = rsrc((char *)L.y + (size_t)c.rank * nb, nb);
    const __amdgpu_buffer_rsrc_t sr = rsrc(L.stats, a.n_ranks * L.stats_stride * 8u);
    // the first pair's residual and weight do not depend on any flag
    const uint32_t e0 = bbeg * NORM_BLOCK + lane * 4u;
    u32x2 r0 = {0u, 0u}, r1 = {0u, 0u}, g0 = {0u, 0u}, g1 = {0u, 0u};
    if (bbeg < bend) {
        r0 = ld8<CP_PLAIN>(resr, e0 * 2u);
        g0 = ld8<CP_PLAIN>(gr, (e0 % L.hidden) * 2u);
        if (bbeg + 1u < bend) {
            r1 = ld8<CP_PLAIN>(resr, (e0 + NORM_BLOCK) * 2u);
            g1 = ld8<CP_PLAIN>(gr, ((e0 + NORM_BLOCK) % L.hidden) * 2u);
        }
    }
    load_seq(a, c);
    const Ctl ctl{a.ctl};
    start_delay(a, c);
    raise_arrival<LOCAL>(a, c);
    bool ok = wait_arrivals<LOCAL>(a, c, ctl);
    mark(c, c.t_sync);
    __amdgpu_buffer_rsrc_t src[NMAX];
#pragma unroll
    for (int s = 0; s < NMAX; ++s)
        src[s] = in_rsrc(a, (uint32_t)s < N ? (uint32_t)s : 0u);
    u32x2 h0 = {0u, 0u}, h1 = {0u, 0u};
    for (uint32_t b = bbeg; ok && b < bend; b += 2u) {
        const bool two = b + 1u < bend;
        const uint32_t e = b * NORM_BLOCK + lane * 4u;
        u32x2 V[NMAX], U[NMAX];
#pragma unroll
        for (int s = 0; s < NMAX; ++s)
            if ((uint32_t)s < N) {
                V[s] = ld8<CP_DEV>(src[s], e * 2u);
                U[s] = two ? ld8<CP_DEV>(src[s], (e + NORM_BLOCK) * 2u) : u32x2{0u, 0u};
            }
        const bool first = b == bbeg;
        const u32x2 rw = first ? r0 : ld8<CP_PLAIN>(resr, e * 2u);
        const u32x2 rw2 = first ? r1 : two ? ld8<CP_PLAIN>(resr, (e + NORM_BLOCK) * 2u)
                                           : u32x2{0u, 0u};
        Acc4 acc, acc2;
#pragma unroll
        for (int s = 0; s < NMAX; ++s)
            if ((uint32_t)s < N) {
                if (s == 0) { acc.init(V[s].x, V[s].y); acc2.init(U[s].x, U[s].y); }
                else { acc.add(V[s].x, V[s].y); acc2.add(U[s].x, U[s].y); }
            }
        u32x2 aw, aw2;
        aw.x = pack_bf16(acc.v[0], acc.v[1]);
        aw.y = pack_bf16(acc.v[2], acc.v[3]);
        aw2.x = pack_bf16(acc2.v[0], acc2.v[1]);
        aw2.y = pack_bf16(acc2.v[2], acc2.v[3]);
        const u32x2 hw = add_round4(aw, rw), hw2 = add_round4(aw2, rw2);
        st8<CP_NT>(hw, oh, e * 2u);
        if (two)
            st8<CP_NT>(hw2, oh, (e + NORM_BLOCK) * 2u);
        if (first) {
            h0 = hw;
            h1 = hw2;
        }
        const float sq = wave_sum(sumsq4(hw));
        const float sq2 = wave_sum(sumsq4(hw2));
        if (lane < (two ? 2u : 1u)) {
            u32x2 en; en.x = __float_as_uint(lane == 0u ? sq : sq2); en.y = c.flag;
            st8<CP_DEV>(en, sr, (c.rank * L.stats_stride + b + lane) * 8u);
        }
    }
    // normalise this wave's blocks (one wait per row they touch)
    const uint32_t B = L.hidden / NORM_BLOCK;
    uint32_t have = 0xFFFFFFFFu;
    float r = 0.0f;
    for (uint32_t b = bbeg; ok && b < bend; ++b) {
        const uint32_t row = b / B;
        if (row != have) {
            if (!row_rinv<LOCAL>(L, c, ctl, sr, row, B, &r)) {
                ok = false;                                    // watchdog: status recorded
                break;
            }
            have = row;
        }
        const uint32_t e = b * NORM_BLOCK + lane * 4u;
        const u32x2 hw = b == bbeg ? h0 : b == bbeg + 1u ? h1 : ld8<CP_PLAIN>(oh, e * 2u);
        const u32x2 gw = b == bbeg ? g0 : b == bbeg + 1u ? g1 : ld8<CP_PLAIN>(gr, (e % L.hidden) * 2u);
        st8<CP_NT>(scale4(hw, gw, r), oy, e * 2u);
    }
    mark(c, c.t_data);
    finish(a, c);
}

// ================================= one-shot DIRECT + add + norm, row-wise
// For batched decode (8 or more rows per rank) a workgroup of 16 waves owns
// one (rank, row): after the arrival flags wave w reduces the row's blocks
// w, w+16, ... in place (8 bytes per lane from every rank's input, both
// blocks of a pair in flight together), adds the residual, writes h and
// puts each block's sum of squares in LDS; the row's sum is then folded in
// LDS and y written -- the stand-alone kernel's structure (norm.hip) with
// the AllReduce in front, so the sums, their order and the bits are the
// same.  No workgroup waits for another's sums.  Rows of up to 8192
// elements (2 blocks per wave, kept in registers: at 50 VGPRs two such
// workgroups fit a CU; with 4 blocks per wave one did, and a batch of 32
// rows took 8.8 us per call instead of 7.6).
constexpr uint32_t ROWS_WAVES = 16;
constexpr uint32_t ROWS_PER_WAVE = 2;

template <int NMAX, bool LOCAL, int HOOKS>
__global__ __launch_bounds__(1024) void k_oneshot_rows_norm(const NormLaunch L)
{
    const Launch &a = L.base;
    __shared__ float bsum[ROWS_WAVES * ROWS_PER_WAVE];
    __shared__ float rinv_s;
    Ctx0 c;
    begin<LOCAL, HOOKS>(a, c);
    const uint32_t N = a.n_ranks;
    const uint32_t row = c.part;                          // one part per row
    const uint32_t lane = threadIdx.x & 63u, wave = threadIdx.x >> 6;
    const uint32_t B = L.hidden / NORM_BLOCK;
    const uint32_t rows = a.n / L.hidden;
    const bool live = row < rows && (blockDim.x >> 6) == ROWS_WAVES;
    const uint32_t nb = a.n * 2u;
    const __amdgpu_buffer_rsrc_t resr = rsrc(L.res[c.rank], nb);
    const __amdgpu_buffer_rsrc_t gr = rsrc(L.gamma, L.hidden * 2u);
    const __amdgpu_buffer_rsrc_t oh = rsrc((char *)a.out + (size_t)c.rank * nb, nb);
    const __amdgpu_buffer_rsrc_t oy = rsrc((char *)L.y + (size_t)c.rank * nb, nb);
    const uint32_t row0 = row * L.hidden;
    // residual and weight need no flag: the waves that do not poll load
    // them before the arrival wait, the polling wave after it
    u32x2 rk[ROWS_PER_WAVE], gk[ROWS_PER_WAVE];
    const bool poller = wave == 0u;
    if (!poller) {
#pragma unroll
        for (int k = 0; k < (int)ROWS_PER_WAVE; ++k) {
            const uint32_t j = wave + ROWS_WAVES * k;
            const uint32_t col = j * NORM_BLOCK + lane * 4u;
            rk[k] = live && j < B ? ld8<CP_PLAIN>(resr, (row0 + col) * 2u) : u32x2{0u, 0u};
            gk[k] = live && j < B ? ld8<CP_PLAIN>(gr, col * 2u) : u32x2{0u, 0u};
        }
    }
    load_seq(a, c);
    const Ctl ctl{a.ctl};
    start_delay(a, c);
    raise_arrival<LOCAL>(a, c);
    if (!wait_arrivals_wg<LOCAL>(a, c, ctl))
        return;                                           // every wave returns here
    mark(c, c.t_sync);
    if (poller) {
#pragma unroll
        for (int k = 0; k < (int)ROWS_PER_WAVE; ++k) {
            const uint32_t j = wave + ROWS_WAVES * k;
            const uint32_t col = j * NORM_BLOCK + lane * 4u;
            rk[k] = live && j < B ? ld8<CP_PLAIN>(resr, (row0 + col) * 2u) : u32x2{0u, 0u};
            gk[k] = live && j < B ? ld8<CP_PLAIN>(gr, col * 2u) : u32x2{0u, 0u};
        }
    }
    __amdgpu_buffer_rsrc_t src[NMAX];
#pragma unroll
    for (int s = 0; s < NMAX; ++s)
        src[s] = in_rsrc(a, (uint32_t)s < N ? (uint32_t)s : 0u);
    u32x2 hk[ROWS_PER_WAVE];
#pragma unroll
    for (int k = 0; k < (int)ROWS_PER_WAVE; k += 2) {
        const uint32_t j = wave + ROWS_WAVES * k, j2 = j + ROWS_WAVES;
        const bool in1 = live && j < B, in2 = live && j2 < B;
        const uint32_t e = row0 + j * NORM_BLOCK + lane * 4u;
        const uint32_t e2 = e + ROWS_WAVES * NORM_BLOCK;
        u32x2 V[NMAX], U[NMAX];
#pragma unroll
        for (int s = 0; s < NMAX; ++s)
            if ((uint32_t)s < N) {
                V[s] = in1 ? ld8<CP_DEV>(src[s], e * 2u) : u32x2{0u, 0u};
                U[s] = in2 ? ld8<CP_DEV>(src[s], e2 * 2u) : u32x2{0u, 0u};
            }
        Acc4 acc, acc2;
#pragma unroll
        for (int s = 0; s < NMAX; ++s)
            if ((uint32_t)s < N) {
                if (s == 0) { acc.init(V[s].x, V[s].y); acc2.init(U[s].x, U[s].y); }
                else { acc.add(V[s].x, V[s].y); acc2.add(U[s].x, U[s].y); }
            }
        u32x2 aw, aw2;
        aw.x = pack_bf16(acc.v[0], acc.v[1]);
        aw.y = pack_bf16(acc.v[2], acc.v[3]);
        aw2.x = pack_bf16(acc2.v[0], acc2.v[1]);
        aw2.y = pack_bf16(acc2.v[2], acc2.v[3]);
        hk[k] = add_round4(aw, rk[k]);
        hk[k + 1] = add_round4(aw2, rk[k + 1]);
        if (in1) {
            st8<CP_NT>(hk[k], oh, e * 2u);
            const float sq = wave_sum(sumsq4(hk[k]));
            if (lane == 0u)
                bsum[j] = sq;
        }
        if (in2) {
            st8<CP_NT>(hk[k + 1], oh, e2 * 2u);
            const float sq = wave_sum(sumsq4(hk[k + 1]));
            if (lane == 0u)
                bsum[j2] = sq;
        }
    }
    __syncthreads();
    if (wave == 0u) {
        // the fold of norm_math.h: lane l holds blocks l, l+64, ... (B <= 32 here)
        const float part = lane < B ? bsum[lane] : 0.0f;
        const float r = rms_inv(wave_sum(part), L.hidden, L.eps);
        if (lane == 0u)
            rinv_s = r;
    }
    __syncthreads();
    const float r = rinv_s;
#pragma unroll
    for (int k = 0; k < (int)ROWS_PER_WAVE; ++k) {
        const uint32_t j = wave + ROWS_WAVES * k;
        if (live && j < B)
            st8<CP_NT>(scale4(hk[k], gk[k], r), oy, (row0 + j * NORM_BLOCK + lane * 4u) * 2u);
    }
    mark(c, c.t_data);
    finish(a, c);
}

// ======================================================= one-shot sentinel
// Push model: rank q writes chunk c of its input into every peer's inbox
// [peer][q][buffer]; each receiver polls its own inbox until no element is
// the sentinel, reduces, and re-arms the slots it consumed.  Inboxes are
// fixed-size windows walked in rounds as in the LL kernel (round j of part p:
// window bytes [1024 p, 1024 (p+1)) of buffer (flag + j) & 1).  The receipt
// of a peer's round-j data proves the peer finished round j-1, re-arm
// included (each round ends with its re-arm stores acknowledged), so the
// re-arm of a buffer always lands before the peer's round j+2 write into it.
//
// As in the one-shot LL kernel, a workgroup of SENT_WAVES = 8 waves owns 64
// chunks (of 8 elements) per round and the peers are split over the waves:
// wave w pushes the chunk into the inboxes of the peers s with s % 8 == w,
// and once those stores are acknowledged it receives the same peers' chunks
// from its own inbox, re-arms their slots and stages the values in LDS;
// after a workgroup barrier wave 0 reduces the tile in global rank order.
// (8 waves rather than 4, same-box A/B: 4 ranks x 8 KiB 2.67 -> 2.46 us,
// 8 x 16 KiB 3.36 -> 2.96, 16 ranks x 112 KiB two-shot 8.9 -> 6.8; the
// 16-rank one-shot 17.3 -> 17.8.)
constexpr int SENT_WAVES = 8;

template <int NMAX, bool F32, bool LOCAL>
__device__ __forceinline__ bool sent_round(const Launch &a, Ctx0 &c, const Ctl &ctl,
                                           __amdgpu_buffer_rsrc_t box,
                                           __amdgpu_buffer_rsrc_t o, uint32_t ch, uint32_t G,
                                           uint32_t rnd, bool more, u32x4 x,
                                           u32x4 (*stage)[64], uint32_t *failed)
{
    constexpr int PW = (NMAX + SENT_WAVES - 1) / SENT_WAVES;
    const uint32_t N = a.n_ranks;
    const uint32_t sb = a.s1_stride;
    const uint32_t lane = threadIdx.x & 63u, wave = threadIdx.x >> 6;
    const bool active = ch < G;
    // inboxes [recv][send][buffer] x s1_stride under one descriptor
    const uint32_t win = (c.part * 64u + lane) * 16u + ((c.flag + rnd) & 1u) * sb;
    auto slot = [&](uint32_t recv, uint32_t send) { return win + ((recv * N + send) * 2u) * sb; };
    uint32_t pend = 0;
#pragma unroll
    for (int j = 0; j < PW; ++j) {
        const uint32_t s = wave + (uint32_t)(SENT_WAVES * j);
        if (s < N && s != c.rank && active)
            pend |= 1u << j;
    }
    const uint32_t mine = pend;
    // push (send) to this wave's peers
#pragma unroll
    for (int j = 0; j < PW; ++j)
        if ((mine >> j) & 1u)
            st16<Pol<LOCAL>::ST>(x, box, slot(wave + (uint32_t)(SENT_WAVES * j), c.rank));
    if (wave == 0u)
        stage[c.rank][lane] = x;
    wait_stores();                  // receive only after the pushes are acknowledged
    // Poll loads are issued by every lane, slots with nothing (left) to
    // receive at OFF_NONE (zeros, no traffic), so the compiler keeps the two
    // polls in flight; a slot goes to the LDS tile as soon as it is seen
    // complete, so nothing after the loop reads a poll register.
    u32x4 A0[PW], A1[PW];
    auto issue = [&](u32x4 *A) {
#pragma unroll
        for (int j = 0; j < PW; ++j)
            A[j] = ld16<Pol<LOCAL>::LD>(box, ((pend >> j) & 1u)
                                                 ? slot(c.rank, wave + (uint32_t)(SENT_WAVES * j))
                                                 : OFF_NONE);
    };
    auto check = [&](const u32x4 *A) {
#pragma unroll
        for (int j = 0; j < PW; ++j)
            if ((pend >> j) & 1u)
                if (sent_ready(A[j])) {
                    pend &= ~(1u << j);
                    stage[wave + SENT_WAVES * j][lane] = A[j];
                }
    };
    Watch w;
    w.begin(a.watchdog_ticks);
    issue(A0);
    while (true) {
        compiler_fence();
        issue(A1);
        check(A0);
        if (!wave_any(pend != 0u))
            break;
        if (w.expired(ctl, c.rank, pend ? wave + SENT_WAVES * first_bit(pend) : 0u, c.call)) {
            *failed = 1u;                           // every wave still meets the barrier
            break;
        }
        compiler_fence();
        issue(A0);
        check(A1);
        if (!wave_any(pend != 0u))
            break;
    }
    mark_once(c, c.t_sync);
    lds_barrier();                  // the tile only: the polls in flight are waited for below
    if (*failed)
        return false;
    if (wave == 0u && active) {
        // every row of the tile at once (rows of absent ranks are not folded)
        u32x4 t[NMAX];
#pragma unroll
        for (int s = 0; s < NMAX; ++s)
            t[s] = stage[s][lane];
        Acc8 acc;
#pragma unroll
        for (int s = 0; s < NMAX; ++s)
            if ((uint32_t)s < N) {
                if (s == 0) acc.init(t[s]); else acc.add(t[s]);
            }
        store8<F32, SENT_OUT>(o, ch * 8u, acc);
    }
    // re-arm what was consumed (resetRange), off the path to the output;
    // the barrier below waits for these stores (and the polls still in
    // flight, whose registers stay reserved until here) before the next
    // round's pushes
#pragma unroll
    for (int k = 0; k < PW; ++k)
        if ((mine >> k) & 1u)
            st16<Pol<LOCAL>::ST>(sentinel4(), box, slot(c.rank, wave + (uint32_t)(SENT_WAVES * k)));
#pragma unroll
    for (int k = 0; k < PW; ++k)
        asm volatile("" ::"v"(A0[k]), "v"(A1[k]));
    // before this part's next round pushes anything, its re-arms are
    // performed: a peer's reuse of these slots follows its receipt of that push
    if (more)
        wait_stores();
    __syncthreads();                                // the tile is reused next round
    return true;
}

template <int NMAX, bool F32, bool LOCAL, int HOOKS>
__global__ __launch_bounds__(512) void k_oneshot_sentinel(const Launch a)
{
    __shared__ u32x4 stage[NMAX][64];
    __shared__ uint32_t failed;
    Ctx0 c;
    begin<LOCAL, HOOKS>(a, c);
    const uint32_t G = a.n >> 3;
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t step = a.parts * 64u;
    const uint32_t rounds = (G + step - 1u) / step;
    const __amdgpu_buffer_rsrc_t inr = in_rsrc(a, c.rank);
    const __amdgpu_buffer_rsrc_t o = out_rsrc(a, c.rank, F32);
    if (threadIdx.x == 0)
        failed = 0u;
    // every wave pushes the chunk, so every wave loads it (the loads meet in L2)
    uint32_t ch = c.part * 64u + lane;
    u32x4 x = ch < G ? ld16<CP_PLAIN>(inr, ch * 16u) : u32x4{0u, 0u, 0u, 0u};
    load_seq(a, c);
    const Ctl ctl{a.ctl};
    const __amdgpu_buffer_rsrc_t box = rsrc(a.s1, a.n_ranks * a.n_ranks * 2u * a.s1_stride);
    start_delay(a, c);
    // round 0 straight-line (see the one-shot LL kernel), later rounds looped
    if (!sent_round<NMAX, F32, LOCAL>(a, c, ctl, box, o, ch, G, 0u, rounds > 1u, x, stage,
                                      &failed))
        return;
    for (uint32_t it = 1; it < rounds; ++it) {
        ch += step;
        x = ch < G ? ld16<CP_PLAIN>(inr, ch * 16u) : u32x4{0u, 0u, 0u, 0u};
        if (!sent_round<NMAX, F32, LOCAL>(a, c, ctl, box, o, ch, G, it, it + 1u < rounds, x, stage,
                                          &failed))
            return;
    }
    mark(c, c.t_data);
    finish(a, c);
}


// ============================================== in-place data phases
// Shared by the flag kernels (DIRECT) and their barrier-ful baselines, so
// that the two differ only in how they synchronise.

// Descriptors of every rank's input, built before a kernel's first wait so
// that reading the input pointers from the launch record is not a round of
// loads between the synchronisation and the first data load.  Slots of
// absent ranks hold null pointers and are only ever addressed past the end.
template <int NMAX>
__device__ __forceinline__ void input_rsrcs(const Launch &a, __amdgpu_buffer_rsrc_t (&src)[NMAX])
{
#pragma unroll
    for (int s = 0; s < NMAX; ++s) {
        src[s] = in_rsrc(a, (uint32_t)s);
        asm volatile("" ::"s"(src[s]));
    }
}

// One-shot: out[rank][8ch .. 8ch+8) = fold over every input, for the
// workgroup's chunks ch = ch0, ch0 + step, ...  Loads are issued
// unconditionally (absent ranks past the end: zeros, no traffic), so the
// compiler keeps the N loads of a chunk in one run instead of waiting for
// earlier loads before each (the load counter is in order).
template <int NMAX, bool F32>
__device__ __forceinline__ void oneshot_data(const Launch &a, const __amdgpu_buffer_rsrc_t (&src)[NMAX],
                                             __amdgpu_buffer_rsrc_t o, uint32_t G, uint32_t ch0,
                                             uint32_t step)
{
    const uint32_t N = a.n_ranks;
    if (a.unit4) {
        // small messages: 4 elements (8 bytes) per lane, so the fold -- a
        // chain of unpack and add instructions issued by one wave -- is
        // half as long per lane (8 x 16 KiB: 0.28 us of the call for 8
        // elements per lane); G counts 4-element units here
        for (uint32_t ch = ch0; ch < G; ch += step) {
            u32x2 V[NMAX];
#pragma unroll
            for (int s = 0; s < NMAX; ++s)
                V[s] = ld8<CP_DEV>(src[s], (uint32_t)s < N ? ch * 8u : OFF_NONE);
            Acc4 acc;
#pragma unroll
            for (int s = 0; s < NMAX; ++s)
                if ((uint32_t)s < N) {
                    if (s == 0) acc.init(V[s].x, V[s].y); else acc.add(V[s].x, V[s].y);
                }
            wait_stores();
            store4<F32, D1_OUT>(o, ch * 4u, acc.v);
        }
        return;
    }
    for (uint32_t ch = ch0; ch < G; ch += step) {
        u32x4 V[NMAX];
#pragma unroll
        for (int s = 0; s < NMAX; ++s)
            V[s] = ld16<CP_DEV>(src[s], (uint32_t)s < N ? ch * 16u : OFF_NONE);
        Acc8 acc;
#pragma unroll
        for (int s = 0; s < NMAX; ++s)
            if ((uint32_t)s < N) {
                if (s == 0) acc.init(V[s]); else acc.add(V[s]);
            }
        wait_stores();                  // every load consumed: the next chunk's run has no waits
        store8<F32, D1_OUT>(o, ch * 8u, acc);
    }
}

// Two-shot: rank q's slice [lo, lo + 8G) of every input, folded in rank
// order and stored into that slice of every rank's output (streaming
// device-scope stores), TS_CPI chunks per lane per round.
constexpr uint32_t TS_CPI = TWOSHOT_DIRECT_CHUNKS;   // chunks per lane per round
// input loads: plain.  The inputs are final before the launch, so no scope
// is needed.  Streaming device-scope loads, taken while the kernel had more
// rounds in its prologue (8 x 4 MiB: 13.20 against 13.27 plain then), now
// cost 0.2-0.8 us per call on most boxes (12.81-12.93 -> 12.01-12.08 us,
// three rounds of fresh processes on each of two boxes; one box within
// noise); without the flags the plain-load data phase runs at 10.86 us per
// call against 10.45 for a plain copy of the same 64 MiB.
constexpr int TS_LD = CP_PLAIN;
constexpr int TS_ST = CP_NT | CP_DEV;               // output stores (streaming)

template <int NMAX, bool F32>
__device__ __forceinline__ void twoshot_data(const Launch &a, const __amdgpu_buffer_rsrc_t (&src)[NMAX],
                                             __amdgpu_buffer_rsrc_t oa, uint32_t lo, uint32_t G,
                                             uint32_t ch0, uint32_t step)
{
    const uint32_t N = a.n_ranks;
    const uint32_t esz = F32 ? 4u : 2u;
    // TS_CPI chunks per lane per round keep more loads in flight (2 measured
    // best at 4 MiB per rank: 1, 3 and 4 lose 6-9%)
    for (uint32_t ch = ch0; ch < G; ch += TS_CPI * step) {
        u32x4 V[TS_CPI][NMAX];
        bool in[TS_CPI];
        uint32_t off[TS_CPI];
#pragma unroll
        for (int k = 0; k < TS_CPI; ++k) {
            in[k] = ch + k * step < G;
            off[k] = in[k] ? (lo + (ch + k * step) * 8u) * 2u : OFF_NONE;
        }
        // all NMAX slots are loaded (those of absent ranks past the end), so
        // that the loads form one straight run the compiler does not split
#pragma unroll
        for (int s = 0; s < NMAX; ++s)
#pragma unroll
            for (int k = 0; k < TS_CPI; ++k)
                V[k][s] = ld16<TS_LD>(src[s], (uint32_t)s < N ? off[k] : OFF_NONE);
        Acc8 acc[TS_CPI];
#pragma unroll
        for (int k = 0; k < TS_CPI; ++k)
#pragma unroll
            for (int s = 0; s < NMAX; ++s)
                if ((uint32_t)s < N) {
                    if (s == 0) acc[k].init(V[k][s]);
                    else acc[k].add(V[k][s]);
                }
        // the round's loads are all consumed (those of absent ranks too), so
        // the next round's loads again issue without waits
        wait_stores();
#pragma unroll
        for (int r = 0; r < NMAX; ++r)
            if ((uint32_t)r < N) {
#pragma unroll
                for (int k = 0; k < TS_CPI; ++k) {
                    const uint32_t o = in[k] ? ((uint32_t)r * a.n + lo + (ch + k * step) * 8u) * esz
                                             : OFF_NONE;
                    if constexpr (F32) {
                        u32x4 l, h;
                        l.x = __float_as_uint(acc[k].v[0]); l.y = __float_as_uint(acc[k].v[1]);
                        l.z = __float_as_uint(acc[k].v[2]); l.w = __float_as_uint(acc[k].v[3]);
                        h.x = __float_as_uint(acc[k].v[4]); h.y = __float_as_uint(acc[k].v[5]);
                        h.z = __float_as_uint(acc[k].v[6]); h.w = __float_as_uint(acc[k].v[7]);
                        st16<TS_ST>(l, oa, o);
                        st16<TS_ST>(h, oa, o + 16u);
                    } else {
                        st16<TS_ST>(acc[k].bf16(), oa, o);
                    }
                }
            }
    }
}

// ========================================================= one-shot DIRECT
// After the arrival flags, each rank reads every peer's input in place
// with device-coherent loads and reduces.  The input of call k must stay
// unchanged until call k has completed on every rank (the application-level
// A/B double buffering of the SiFAR page, "SiFAR：无同步All-Reduce技术突破低
// 延迟LLM推理瓶颈", technique one).
template <int NMAX, bool F32, bool LOCAL, int HOOKS>
__global__ __launch_bounds__(256) void k_oneshot_direct(const uint32_t arr, const Launch a)
{
    raise_arrival_first<LOCAL, HOOKS>(arr);
    Ctx0 c;
    begin<LOCAL, HOOKS>(a, c);
    const uint32_t G = a.unit4 ? a.n >> 2 : a.n >> 3;          // lane units of 4 or 8 elements
    const uint32_t step = a.parts * blockDim.x;
    load_seq(a, c);
    const Ctl ctl{a.ctl};
    start_delay(a, c);
    raise_arrival_late<LOCAL, HOOKS>(a, c);
    __amdgpu_buffer_rsrc_t src[NMAX];
    input_rsrcs<NMAX>(a, src);
    const __amdgpu_buffer_rsrc_t o = out_rsrc(a, c.rank, F32);
    if (!wait_arrivals<LOCAL>(a, c, ctl))
        return;
    mark(c, c.t_sync);
    oneshot_data<NMAX, F32>(a, src, o, G, c.part * blockDim.x + threadIdx.x, step);
    mark(c, c.t_data);
    finish(a, c);
}

// ========================================================= two-shot DIRECT
// Reduce-scatter: rank q reads slice q of every rank's input in place (after
// the arrival flags) and reduces it; all-gather: it stores the bf16
// result straight into slice q of every rank's output (the bcast of the
// reduced value), with streaming device-scope stores.  Each workgroup then
// waits for its stores to be acknowledged and raises its completion flag;
// one workgroup per rank waits for every writer's flag, after which every
// slice of that rank's output is known to be complete.
// Moves exactly the algorithmic bytes: N inputs read once, N outputs written
// once.
template <int NMAX, bool F32, bool LOCAL, int HOOKS>
__global__ __launch_bounds__(256) void k_twoshot_direct(const uint32_t arr, const Launch a)
{
    raise_arrival_first<LOCAL, HOOKS>(arr);
    // The first arrival poll goes out with the launch record's loads: most
    // workgroups of this large grid start after the arrival writers (parts
    // 0..7, dispatched first), so it usually finds the flags and saves a
    // poll round trip (8 x 4 MiB: 12.08-12.09 -> 11.97-12.06 us per call).
    // The one-shot kernels start all their workgroups at once; there an
    // early poll meets the line before the writers' stores have put it in
    // the L2 and costs a memory round trip (8 x 16 KiB 2.18 -> 2.35 us).
    uint32_t early = 0;
    if constexpr (LOCAL)
        early = early_arrival_poll();
    Ctx0 c;
    begin<LOCAL, HOOKS>(a, c);
    const uint32_t N = a.n_ranks;
    const uint32_t q = c.rank;
    const uint32_t L = a.slice;
    const uint32_t lo = q * L;
    const uint32_t Lq = lo >= a.n ? 0u : (a.n - lo < L ? a.n - lo : L);
    const uint32_t G = Lq >> 3;                     // chunks of my slice
    const uint32_t step = a.parts * blockDim.x;
    load_seq(a, c);
    const Ctl ctl{a.ctl};
    start_delay(a, c);
    raise_arrival_late<LOCAL, HOOKS>(a, c);
    // Every input is read after the arrival wait, the rank's own too: with
    // the prologue down to one launch-record round and the sequence load,
    // the flags arrive about when loads could first be issued, and loading
    // the own chunks ahead of the wait measured slower (8 x 4 MiB: 12.39 vs
    // 12.64 us per call).
    __amdgpu_buffer_rsrc_t src[NMAX];
    input_rsrcs<NMAX>(a, src);
    const __amdgpu_buffer_rsrc_t oa = out_all(a, F32);
    if (!wait_arrivals_wg<LOCAL>(a, c, ctl, LOCAL ? &early : nullptr))
        return;
    mark(c, c.t_sync);
    twoshot_data<NMAX, F32>(a, src, oa, lo, G, c.part * blockDim.x + threadIdx.x, step);
    mark(c, c.t_data);
    // completion: my stores are at the coherence point, then my flag.  The
    // flags of the writers on one XCD (parts p with p % 8 == x) are packed
    // together: writer (s, p) owns word x*N*P8 + s*P8 + p/8, P8 = ceil(parts/8).
    // One waiter per rank and XCD -- a part of the last block, which streams
    // last, so polling (reads of freshly written lines, which slow the other
    // writers' streams) is short -- waits for all flags of its XCD; together
    // the waiters of rank q see every writer, which proves that every slice
    // of q's output is complete before q's workgroups exit.
    wait_stores();
    __syncthreads();
    const uint32_t P8 = (a.parts + XCDS - 1u) / XCDS;
    const __amdgpu_buffer_rsrc_t dn = rsrc(a.done, MAX_RANKS * DONE_STRIDE * 4u);
    if (threadIdx.x == 0)
        st4<Pol<LOCAL>::ST>(c.flag, dn, ((c.part % XCDS) * N * P8 + q * P8 + c.part / XCDS) * 4u);
    const bool waiter = a.parts % (uint32_t)XCDS == 0u ? c.part >= a.parts - (uint32_t)XCDS
                                                       : c.part < (uint32_t)XCDS;
    if (waiter && threadIdx.x < 64u) {
        const uint32_t lane = threadIdx.x;
        const uint32_t x = c.part % XCDS;
        const uint32_t per = (a.parts - x + XCDS - 1u) / XCDS;   // parts x, x+8, ...
        const uint32_t total = N * per;                // writers this waiter covers
        const uint32_t base = x * N * P8;
        Watch w;
        w.begin(a.watchdog_ticks);
        // each lane waits for its share of the writers in turn, two polls of
        // the word in flight: while one value is checked the next is on its way
        for (uint32_t i = lane; i < total; i += 64u) {
            const uint32_t off = (base + (i / per) * P8 + i % per) * 4u;
            uint32_t v0 = ld4<Pol<LOCAL>::LD>(dn, off), v1;
            while (true) {
                compiler_fence();
                v1 = ld4<Pol<LOCAL>::LD>(dn, off);
                if ((int32_t)(v0 - c.flag) >= 0)
                    break;
                if (w.expired(ctl, q, i / per, c.call))
                    return;
                compiler_fence();
                v0 = ld4<Pol<LOCAL>::LD>(dn, off);
                if ((int32_t)(v1 - c.flag) >= 0)
                    break;
            }
        }
    }
    finish(a, c);
}

// ============================================================ barrier-ful
// The classic structure the flag protocols replace ([EMC] "全局内存屏障": a
// global barrier before the reads, so every rank's data is ready, and one
// after the writes, so no rank overwrites a buffer a peer still reads).  It
// is a measured baseline: the same reads, fold and writes as the DIRECT
// kernels, with both synchronisations done by device-wide barriers over all
// ranks' workgroups instead of flags.
//
// Barrier (two levels, so that no single counter takes every arrival):
// workgroup b arrives at the counter of its group b % 8 -- one XCD, since
// dispatch is round-robin; the last arrival of a group resets that counter
// and arrives at the group counter; the last group resets it and publishes
// the call's flag into the barrier's generation word, one copy per group;
// every other workgroup polls its group's copy.  Flags grow monotonically,
// so generation words need no reset.
// It is a rendezvous only: nothing written inside the kernel before a barrier
// is read by another workgroup after it (inputs are final before the launch,
// outputs are read after it), so no cache write-back or invalidate is needed;
// device-scope atomics order the counters.  (With agent-scope fences around
// each arrival, as a barrier that publishes data needs, measured costs rise
// from 2.5 to 6 us per 16 KiB call and from 5 to 40 us per 4 MiB call.)  The host keeps the grid within
// half the device's resident capacity, so every workgroup runs at once; the
// watchdog bounds the wait otherwise.
__device__ __forceinline__ bool grid_barrier(const Launch &a, const Ctx0 &c, const Ctl &ctl,
                                             uint32_t gen_base)
{
    wait_stores();
    __syncthreads();
    __shared__ uint32_t ok;
    if (threadIdx.x == 0) {
        const uint32_t G = a.parts * a.n_ranks;
        const uint32_t grp = linear_id(a) % (uint32_t)XCDS;
        const uint32_t groups = G < (uint32_t)XCDS ? G : (uint32_t)XCDS;
        const uint32_t size = (G - grp + XCDS - 1u) / XCDS;     // workgroups in my group
        uint32_t *gcnt = a.ctl + CTL_BAR_GROUP + 32u * grp;
        uint32_t *cnt = a.ctl + CTL_BAR_COUNT;
        uint32_t good = 1;
        bool last = false;
        if (__hip_atomic_fetch_add(gcnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
            size - 1u) {
            // counters are reset before anyone can pass this barrier: each
            // reset is acknowledged (performed device-wide) before the next
            // atomic is issued
            __hip_atomic_store(gcnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            wait_stores();
            if (__hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                groups - 1u) {
                __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                wait_stores();
                for (uint32_t x = 0; x < (uint32_t)XCDS; ++x)
                    __hip_atomic_store(a.ctl + gen_base + 32u * x, c.flag, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
                last = true;
            }
        }
        if (!last) {
            uint32_t *gen = a.ctl + gen_base + 32u * grp;
            Watch w;
            w.begin(a.watchdog_ticks);
            while ((int32_t)(__hip_atomic_load(gen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) -
                             c.flag) < 0) {
                if (w.expired(ctl, c.rank, 0u, c.call)) {
                    good = 0;
                    break;
                }
                __builtin_amdgcn_s_sleep(1);
            }
        }
        ok = good;
    }
    __syncthreads();
    return ok != 0u;
}

// One-shot: top barrier, every rank reads all N inputs in place and writes
// its copy, bottom barrier.
template <int NMAX, bool F32, bool LOCAL, int HOOKS>
__global__ __launch_bounds__(256) void k_oneshot_barrier(const Launch a)
{
    Ctx0 c;
    begin<LOCAL, HOOKS>(a, c);
    const uint32_t G = a.unit4 ? a.n >> 2 : a.n >> 3;          // lane units of 4 or 8 elements
    const uint32_t step = a.parts * blockDim.x;
    load_seq(a, c);
    const Ctl ctl{a.ctl};
    start_delay(a, c);
    __amdgpu_buffer_rsrc_t src[NMAX];
    input_rsrcs<NMAX>(a, src);
    const __amdgpu_buffer_rsrc_t o = out_rsrc(a, c.rank, F32);
    if (!grid_barrier(a, c, ctl, CTL_BAR_TOP))
        return;
    mark(c, c.t_sync);
    oneshot_data<NMAX, F32>(a, src, o, G, c.part * blockDim.x + threadIdx.x, step);
    mark(c, c.t_data);
    if (!grid_barrier(a, c, ctl, CTL_BAR_BOTTOM))
        return;
    finish(a, c);
}

// Two-shot: top barrier, rank q reduces slice q of all inputs in place and
// writes it into every rank's output, bottom barrier (every output complete).
template <int NMAX, bool F32, bool LOCAL, int HOOKS>
__global__ __launch_bounds__(256) void k_twoshot_barrier(const Launch a)
{
    Ctx0 c;
    begin<LOCAL, HOOKS>(a, c);
    const uint32_t q = c.rank;
    const uint32_t L = a.slice;
    const uint32_t lo = q * L;
    const uint32_t Lq = lo >= a.n ? 0u : (a.n - lo < L ? a.n - lo : L);
    const uint32_t G = Lq >> 3;
    const uint32_t step = a.parts * blockDim.x;
    load_seq(a, c);
    const Ctl ctl{a.ctl};
    start_delay(a, c);
    __amdgpu_buffer_rsrc_t src[NMAX];
    input_rsrcs<NMAX>(a, src);
    const __amdgpu_buffer_rsrc_t oa = out_all(a, F32);
    if (!grid_barrier(a, c, ctl, CTL_BAR_TOP))
        return;
    mark(c, c.t_sync);
    twoshot_data<NMAX, F32>(a, src, oa, lo, G, c.part * blockDim.x + threadIdx.x, step);
    mark(c, c.t_data);
    if (!grid_barrier(a, c, ctl, CTL_BAR_BOTTOM))
        return;
    finish(a, c);
}

// ============================================================ LL128 lines
// Lane mapping of a line group (480 elements, 1024 bytes): see ar_proto.h.
// A workgroup of 4 waves handles GW line groups per batch, one per
// publishing wave: the wave publishes its group's payload, waits for the
// acknowledgement, then stores the line flags.  The receive is split over
// the waves as in the LL and sentinel kernels: wave w takes every group of
// the batch from the peers s with s % 4 == w, polling their line flags
// together and then loading the payloads.
// Line groups per batch (GW) is a template parameter chosen by the host per
// call: small batches spread a message over more workgroups (more of the
// chip, shorter serial chains), large ones amortise the per-batch hops on
// big messages (measured at 8 ranks: one-shot 16-64 KiB best with 1 group
// per batch, 256-512 KiB with 2; two-shot up to 1 MiB with 1, from 2 MiB
// with 4).  At most 2 above 8 ranks (LDS tile budget).
constexpr int L128_WAVES = 4;

// Cache policies and the arrival-wait form of the LL128 kernels, measured at
// 8 x 512 KiB and 8 x 4 MiB (graphs, same box): non-temporal output stores
// (see LL_OUT) cut the 512 KiB one-shot 8.29 -> 7.84 us, the 512 KiB
// two-shot 4.95 -> 4.66 and the 4 MiB two-shot 24.2 -> 20.8; streaming
// device-scope ones slow the 512 KiB two-shot to 5.2 (they wait for memory
// inside the launch).  Non-temporal staging stores slow every line-protocol
// call (512 KiB two-shot 5.62): the peers' polls then miss the L2.
// Streaming reduce-scatter loads and a single polling wave per workgroup
// move both within 1%.
constexpr int L128_OUT1 = CP_NT;        // one-shot output stores
constexpr int L128_OUT2 = CP_NT;        // two-shot output stores
constexpr bool L128_ARRIVE_WG = false;  // two-shot arrival wait: one polling wave per workgroup
constexpr int L128_RS_LD = CP_DEV;      // two-shot in-place reduce-scatter loads

// reads 8 (or 4) elements of a bf16 buffer at element `e`
template <int CP = CP_PLAIN>
__device__ __forceinline__ u32x4 ld_elems(__amdgpu_buffer_rsrc_t r, uint32_t e, bool half)
{
    if (half) {
        u32x2 p = ld8<CP>(r, e * 2u);
        u32x4 v; v.x = p.x; v.y = p.y; v.z = 0u; v.w = 0u;
        return v;
    }
    return ld16<CP>(r, e * 2u);
}

// The payload store covers the whole 128-byte line: the flag lane writes its
// 8 payload bytes and zeros over the flag slot.  A store of part of a line
// the L2 does not hold makes it fetch the line from memory first (8 x 4 MiB
// two-shot: 4.7 MiB of extra reads per launch, the whole staging footprint);
// a whole-line store needs no fetch, and the flag store that follows finds
// the line in the L2.  A zero flag slot never validates ({f, ~f} needs the
// second word to be the complement of the first).
template <bool LOCAL>
__device__ __forceinline__ void l128_store_payload(__amdgpu_buffer_rsrc_t dst, uint32_t off,
                                                   bool half, u32x4 payload)
{
    if (half) {
        payload.z = 0u;
        payload.w = 0u;
    }
    st16<Pol<LOCAL>::ST>(payload, dst, off);
}

template <bool LOCAL>
__device__ __forceinline__ void l128_store_flag(__amdgpu_buffer_rsrc_t dst, uint32_t off,
                                                uint32_t flag)
{
    u32x2 f; f.x = flag; f.y = ~flag;
    st8<Pol<LOCAL>::ST>(f, dst, off + 8u);
}

__device__ __forceinline__ bool l128_flag_ok(u32x2 f, uint32_t flag)
{
    return f.x == flag && f.y == ~flag;
}

// Receives the GW line groups g[k] (valid when bit k of gvalid; staged in
// window slots slot0 + k of buffer `par`) from this wave's peers
// s = wave + 4j (PW slots; bit j of pmask marks a real peer):
// flag lanes poll the line flags of every (group, peer) still pending, the
// wave votes, then every lane loads its payloads into V[k][j].  lim[j] is
// the number of valid elements of peer j in group index space; a line is
// polled only if one of its elements is valid.  Returns false on watchdog
// expiry.
template <int GW, int PW, bool LOCAL>
__device__ __forceinline__ bool l128_recv(__amdgpu_buffer_rsrc_t reg, uint32_t rb, uint32_t par,
                                          uint32_t slot0, const uint32_t *g, uint32_t gvalid,
                                          uint32_t pmask,
                                          uint32_t wave, uint32_t lane, const L128Lane &ln,
                                          const uint32_t *lim, uint32_t flag, const Ctl &ctl,
                                          uint32_t rank, uint32_t call, uint32_t budget,
                                          u32x4 (*V)[PW])
{
    // peer s's lines of group k: reg + (s*2 + par)*rb + (slot0 + k)*1024 + lane*16
    auto off = [&](int k, int j) {
        return ((wave + (uint32_t)(L128_WAVES * j)) * 2u + par) * rb +
               (slot0 + (uint32_t)k) * L128_BYTES + lane * 16u;
    };
    // Flag polls and payload loads are issued by every lane for every
    // (group, peer) slot, those with nothing to read at OFF_NONE (zeros, no
    // traffic): under per-slot branches each load waited for the one before
    // (8 x 512 KiB: two-shot 5.23 -> 4.78 us, one-shot 9.45 -> 8.74; 8 x 4 MiB
    // two-shot 27.6 -> 24.1).  A half lane reads its whole 16-byte slot (its
    // 8 payload bytes, then the line flag) and clears the upper half.
    uint32_t pend[GW];
    u32x2 F[GW][PW];
    Watch w;
    w.begin(budget);
#pragma unroll
    for (int k = 0; k < GW; ++k) {
        pend[k] = 0;
        const uint32_t line_first = g[k] * L128_ELEMS + 56u * (lane >> 3);
#pragma unroll
        for (int j = 0; j < PW; ++j) {
            const bool need = ((gvalid >> k) & 1u) && ((pmask >> j) & 1u) && ln.half &&
                              line_first < lim[j];
            F[k][j] = ld8<Pol<LOCAL>::LD>(reg, need ? off(k, j) + 8u : OFF_NONE);
            if (need)
                pend[k] |= 1u << j;
        }
    }
    while (true) {
        uint32_t any = 0;
#pragma unroll
        for (int k = 0; k < GW; ++k) {
#pragma unroll
            for (int j = 0; j < PW; ++j)
                if ((pend[k] >> j) & 1u)
                    if (l128_flag_ok(F[k][j], flag))
                        pend[k] &= ~(1u << j);
            any |= pend[k];
        }
        if (!wave_any(any != 0u))
            break;
        if (w.expired(ctl, rank, any ? wave + L128_WAVES * first_bit(any) : 0u, call))
            return false;
        compiler_fence();
#pragma unroll
        for (int k = 0; k < GW; ++k)
#pragma unroll
            for (int j = 0; j < PW; ++j)
                F[k][j] = ld8<Pol<LOCAL>::LD>(reg, ((pend[k] >> j) & 1u) ? off(k, j) + 8u : OFF_NONE);
    }
    // every needed line is complete: load the payloads
    compiler_fence();
#pragma unroll
    for (int k = 0; k < GW; ++k) {
        const uint32_t e = g[k] * L128_ELEMS + ln.elem;
#pragma unroll
        for (int j = 0; j < PW; ++j) {
            const bool need = ((gvalid >> k) & 1u) && ((pmask >> j) & 1u) && e < lim[j];
            V[k][j] = ld16<Pol<LOCAL>::LD>(reg, need ? off(k, j) : OFF_NONE);
            if (ln.half) {
                V[k][j].z = 0u;
                V[k][j].w = 0u;
            }
        }
    }
    return true;
}


template <bool F32, int CP = CP_PLAIN>
__device__ __forceinline__ void store_lane(__amdgpu_buffer_rsrc_t o, uint32_t e, bool half,
                                           const Acc8 &acc)
{
    if (half) store4<F32, CP>(o, e, acc.v); else store8<F32, CP>(o, e, acc);
}

// ====================================================== one-shot LL128
// Rank r publishes its whole input as line groups.  Batch j of a workgroup
// covers groups (part + j*parts)*GW + k, k < GW; wave k < GW publishes
// group k.  Every wave receives the batch from its peers into an LDS tile
// [N][GW][64 lanes]; after a workgroup barrier each publishing wave reduces
// its group in global rank order and writes it.  Staging is a fixed window
// per rank walked in rounds (one batch per part per round) as in the LL
// kernel: batch j of part p sits in window slots p*GW .. p*GW + GW-1 of
// buffer (flag + j) & 1 with flag flag + j, and the workgroup barrier after
// a batch's receive (every wave has received it) comes before the next
// batch's publish, which is the double buffer's permit.
template <int NMAX, bool F32, bool LOCAL, int GW, int HOOKS>
__global__ __launch_bounds__(256) void k_oneshot_ll128(const Launch a)
{
    constexpr int PW = (NMAX + L128_WAVES - 1) / L128_WAVES;
    __shared__ u32x4 stage[NMAX][GW][64];
    __shared__ uint32_t failed;
    Ctx0 c;
    begin<LOCAL, HOOKS>(a, c);
    const uint32_t N = a.n_ranks;
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t wave = threadIdx.x >> 6;
    const uint32_t groups = (a.n + L128_ELEMS - 1u) / L128_ELEMS;
    const uint32_t batches = (groups + GW - 1u) / GW;
    load_seq(a, c);
    const Ctl ctl{a.ctl};
    const L128Lane ln = l128_lane(lane);
    const __amdgpu_buffer_rsrc_t inr = in_rsrc(a, c.rank);
    const __amdgpu_buffer_rsrc_t o = out_rsrc(a, c.rank, F32);
    const uint32_t rb = a.l128_stride;
    const __amdgpu_buffer_rsrc_t reg = rsrc(a.l128, N * 2u * rb);
    const uint32_t slot0 = c.part * (uint32_t)GW;  // this part's window slots
    uint32_t pmask = 0, lim[PW];
#pragma unroll
    for (int j = 0; j < PW; ++j) {
        const uint32_t s = wave + (uint32_t)(L128_WAVES * j);
        lim[j] = a.n;
        if (s < N && s != c.rank)
            pmask |= 1u << j;
    }
    if (threadIdx.x == 0)
        failed = 0u;
    start_delay(a, c);

    // Batches are pipelined across rounds: the input of batch j+1 is loaded
    // while batch j is received, and batch j+1 is published as soon as the
    // workgroup has received batch j (its permit), before batch j is reduced
    // (8 x 512 KiB 7.58 -> 7.19 us, 8 x 16 KiB 3.14 -> 2.89, 8 x 1 MiB
    // 13.3 -> 12.45).  (Written without lambdas: a lambda form changed the
    // compiled two-shot kernel too and cost it 4%.)
    uint32_t b = c.part;
    uint32_t g[GW];
    uint32_t gvalid = 0;
#pragma unroll
    for (int k = 0; k < GW; ++k) {
        g[k] = b * GW + (uint32_t)k;
        if (b < batches && g[k] < groups)
            gvalid |= 1u << k;
    }
    bool pub = wave < (uint32_t)GW && ((gvalid >> wave) & 1u);
    uint32_t em = (b * GW + wave) * L128_ELEMS + ln.elem;
    const uint32_t my_slot = (slot0 + wave) * L128_BYTES + lane * 16u;
    if (pub) {
        u32x4 x = {0u, 0u, 0u, 0u};
        if (em < a.n)
            x = ld_elems(inr, em, ln.half);
        const uint32_t lo = (c.rank * 2u + (c.flag & 1u)) * rb + my_slot;
        l128_store_payload<LOCAL>(reg, lo, ln.half, x);
        wait_stores();
        if (ln.half)
            l128_store_flag<LOCAL>(reg, lo, c.flag);
        stage[c.rank][wave][lane] = x;
    }
    uint32_t rnd = 0;
    for (; b < batches; b += a.parts, ++rnd) {
        const uint32_t fj = c.flag + rnd, bj = fj & 1u;      // this round's flag and buffer
        // the next batch: its input is on its way during this receive
        const uint32_t bn = b + a.parts;
        const bool pubn = wave < (uint32_t)GW && bn < batches && bn * GW + wave < groups;
        const uint32_t emn = (bn * GW + wave) * L128_ELEMS + ln.elem;
        u32x4 xn = {0u, 0u, 0u, 0u};
        if (pubn && emn < a.n)
            xn = ld_elems(inr, emn, ln.half);
        // receive the batch from this wave's peers
        u32x4 V[GW][PW];
        if (!l128_recv<GW, PW, LOCAL>(reg, rb, bj, slot0, g, gvalid, pmask, wave, lane, ln, lim,
                                      fj, ctl, c.rank, c.call, a.watchdog_ticks, V))
            failed = 1u;                            // every wave still meets the barrier
        mark_once(c, c.t_sync);
#pragma unroll
        for (int k = 0; k < GW; ++k)
            if ((gvalid >> k) & 1u)
#pragma unroll
                for (int j = 0; j < PW; ++j)
                    if ((pmask >> j) & 1u)
                        stage[wave + L128_WAVES * j][k][lane] = V[k][j];
        lds_barrier();
        if (failed)
            return;
        // every wave has received this batch: the next one may be published
        if (pubn) {
            const uint32_t lo = (c.rank * 2u + ((fj + 1u) & 1u)) * rb + my_slot;
            l128_store_payload<LOCAL>(reg, lo, ln.half, xn);
            wait_stores();
            if (ln.half)
                l128_store_flag<LOCAL>(reg, lo, fj + 1u);
        }
        if (pub && em < a.n) {
            // every row of the tile at once (rows of absent ranks are not folded)
            u32x4 t[NMAX];
#pragma unroll
            for (int s = 0; s < NMAX; ++s)
                t[s] = stage[s][wave][lane];
            Acc8 acc;
#pragma unroll
            for (int s = 0; s < NMAX; ++s)
                if ((uint32_t)s < N) {
                    if (s == 0) acc.init(t[s]); else acc.add(t[s]);
                }
            store_lane<F32, L128_OUT1>(o, em, ln.half, acc);
        }
        lds_barrier();                              // the tile is reused next batch
        if (pubn)
            stage[c.rank][wave][lane] = xn;
        gvalid = 0;
#pragma unroll
        for (int k = 0; k < GW; ++k) {
            g[k] = bn * GW + (uint32_t)k;
            if (bn < batches && g[k] < groups)
                gvalid |= 1u << k;
        }
        pub = pubn;
        em = emn;
    }
    mark(c, c.t_data);
    finish(a, c);
}

// ====================================================== two-shot LL128
// Reduce-scatter: rank q reduces slice q (elements [q*L, q*L + Lq)) reading
// every rank's input in place after the arrival flags, and publishes the
// bf16 result as line groups.  All-gather: rank q receives every slice's
// groups (its own from registers) and writes them to out[q].  Batches,
// publishing waves and the staging window as in the one-shot kernel; wave w
// receives the batch of the slices of the peers s with s % 4 == w straight
// into out[q], and the waves meet at a barrier before the next batch is
// published (its permit: every wave has received this batch).
template <int NMAX, bool F32, bool LOCAL, int GW, int HOOKS>
__global__ __launch_bounds__(256) void k_twoshot_ll128(const Launch a)
{
    constexpr int PW = (NMAX + L128_WAVES - 1) / L128_WAVES;
    Ctx0 c;
    begin<LOCAL, HOOKS>(a, c);
    const uint32_t N = a.n_ranks;
    const uint32_t q = c.rank;
    const uint32_t L = a.slice;
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t wave = threadIdx.x >> 6;
    const uint32_t groups = (L + L128_ELEMS - 1u) / L128_ELEMS;
    const uint32_t batches = (groups + GW - 1u) / GW;
    load_seq(a, c);
    const Ctl ctl{a.ctl};
    const L128Lane ln = l128_lane(lane);
    start_delay(a, c);
    raise_arrival<LOCAL>(a, c);
    __amdgpu_buffer_rsrc_t src[NMAX];
    input_rsrcs<NMAX>(a, src);
    if (!(L128_ARRIVE_WG ? wait_arrivals_wg<LOCAL>(a, c, ctl) : wait_arrivals<LOCAL>(a, c, ctl)))
        return;
    mark(c, c.t_sync);
    auto slice_len = [&](uint32_t s) -> uint32_t {
        const uint32_t lo = s * L;
        return (s >= N || lo >= a.n) ? 0u : (a.n - lo < L ? a.n - lo : L);
    };
    const uint32_t Lq = slice_len(q);
    const __amdgpu_buffer_rsrc_t o = out_rsrc(a, q, F32);
    const uint32_t rb = a.l128_stride;
    const __amdgpu_buffer_rsrc_t reg = rsrc(a.l128, N * 2u * rb);
    const uint32_t slot0 = c.part * (uint32_t)GW;  // this part's window slots
    uint32_t pmask = 0, lim[PW];
#pragma unroll
    for (int j = 0; j < PW; ++j) {
        const uint32_t s = wave + (uint32_t)(L128_WAVES * j);
        lim[j] = slice_len(s);
        if (s < N && s != q)
            pmask |= 1u << j;
    }

    uint32_t rnd = 0;
    for (uint32_t b = c.part; b < batches; b += a.parts, ++rnd) {
        const uint32_t fj = c.flag + rnd, bj = fj & 1u;      // this round's flag and buffer
        const uint32_t mine_off = (q * 2u + bj) * rb;
        if (rnd > 0u)
            lds_barrier();          // every wave has received the previous batch: the permit
        uint32_t g[GW];
        uint32_t gvalid = 0;
#pragma unroll
        for (int k = 0; k < GW; ++k) {
            g[k] = b * GW + (uint32_t)k;
            if (g[k] < groups)
                gvalid |= 1u << k;
        }
        // ---- reduce-scatter of this wave's group, publish, own copy
        const bool pub = wave < (uint32_t)GW && ((gvalid >> wave) & 1u);
        const uint32_t gm = b * GW + wave;
        const uint32_t em = gm * L128_ELEMS + ln.elem;
        if (pub) {
            u32x4 red = {0u, 0u, 0u, 0u};
            if (em < Lq) {
                // one straight run of loads (absent ranks past the end); a
                // half lane's 4 elements are the upper half of the 16 bytes
                // that end with them (its element index is at least 56, so
                // the load starts inside the buffer and ends where they end)
                const uint32_t eo = (q * L + em - (ln.half ? 4u : 0u)) * 2u;
                u32x4 V[NMAX];
#pragma unroll
                for (int s = 0; s < NMAX; ++s)
                    V[s] = ld16<L128_RS_LD>(src[s], (uint32_t)s < N ? eo : OFF_NONE);
                if (ln.half) {
#pragma unroll
                    for (int s = 0; s < NMAX; ++s) {
                        V[s].x = V[s].z;
                        V[s].y = V[s].w;
                        V[s].z = 0u;
                        V[s].w = 0u;
                    }
                }
                Acc8 acc;
#pragma unroll
                for (int s = 0; s < NMAX; ++s)
                    if ((uint32_t)s < N) {
                        if (s == 0) acc.init(V[s]); else acc.add(V[s]);
                    }
                if constexpr (F32) {
                    // debug path: the owner writes its slice's accumulators to every copy
                    for (uint32_t r = 0; r < N; ++r)
                        store_lane<true>(out_all(a, true), r * a.n + q * L + em, ln.half, acc);
                } else {
                    red = acc.bf16();
                    if (ln.half) {
                        u32x2 p; p.x = red.x; p.y = red.y;
                        st8<L128_OUT2>(p, o, (q * L + em) * 2u);
                    } else {
                        st16<L128_OUT2>(red, o, (q * L + em) * 2u);
                    }
                }
            }
            if constexpr (!F32) {
                const uint32_t lo = mine_off + (slot0 + wave) * L128_BYTES + lane * 16u;
                l128_store_payload<LOCAL>(reg, lo, ln.half, red);
                wait_stores();
                if (ln.half)
                    l128_store_flag<LOCAL>(reg, lo, fj);
            }
        }
        if constexpr (F32)
            continue;
        // ---- all-gather of the batch from this wave's peers
        u32x4 V[GW][PW];
        if (!l128_recv<GW, PW, LOCAL>(reg, rb, bj, slot0, g, gvalid, pmask, wave, lane, ln, lim,
                                      fj, ctl, q, c.call, a.watchdog_ticks, V))
            return;
#pragma unroll
        for (int k = 0; k < GW; ++k) {
            if (!((gvalid >> k) & 1u))
                continue;
            const uint32_t e = g[k] * L128_ELEMS + ln.elem;
#pragma unroll
            for (int j = 0; j < PW; ++j) {
                const uint32_t s = wave + (uint32_t)(L128_WAVES * j);
                if (((pmask >> j) & 1u) && e < lim[j]) {
                    if (ln.half) {
                        u32x2 p; p.x = V[k][j].x; p.y = V[k][j].y;
                        st8<L128_OUT2>(p, o, (s * L + e) * 2u);
                    } else {
                        st16<L128_OUT2>(V[k][j], o, (s * L + e) * 2u);
                    }
                }
            }
        }
    }
    mark(c, c.t_data);
    finish(a, c);
}

// ==================================================== two-shot sentinel
// Reduce-scatter: rank q pushes chunk c of its slice-s part into inbox
// RS[s][q]; rank s polls RS[s][*], reduces in rank order, re-arms.
// All-gather: rank q pushes its reduced chunk into AG[r][q] of every peer r
// and writes it to out[q]; every rank polls AG[q][*], copies to out, re-arms.
// Inbox regions [recv][send][buffer] x s2_stride, one descriptor each:
// fixed-size windows walked in rounds as in the one-shot kernels (round j of
// part p: window bytes [1024 p, 1024 (p+1)) of buffer (flag + j) & 1), every
// round ending with its re-arm stores acknowledged before the next round's
// pushes.
//
// A workgroup of SENT_WAVES waves owns 64 chunks of every slice per round,
// and the peers are split over the waves as in the one-shot kernels: wave w
// pushes the slices of, and receives from, the peers s with s % 8 == w.  The
// received slice-q chunks are staged in LDS and reduced by wave 0, which
// puts the bf16 result in LDS for every wave's all-gather pushes.
template <int NMAX, bool F32, bool LOCAL>
__device__ __forceinline__ bool ts_round(const Launch &a, Ctx0 &c, const Ctl &ctl,
                                         __amdgpu_buffer_rsrc_t inq, __amdgpu_buffer_rsrc_t rsr,
                                         __amdgpu_buffer_rsrc_t agr, __amdgpu_buffer_rsrc_t oa,
                                         uint32_t ch, uint32_t rnd, bool more, u32x4 (*stage)[64],
                                         u32x4 *red, uint32_t *failed)
{
    constexpr int PW = (NMAX + SENT_WAVES - 1) / SENT_WAVES;
    const uint32_t N = a.n_ranks;
    const uint32_t q = c.rank;
    const uint32_t L = a.slice;
    const uint32_t sb = a.s2_stride;
    const uint32_t lane = threadIdx.x & 63u, wave = threadIdx.x >> 6;
    const uint32_t e = ch * 8u;                     // element offset inside a slice
    const uint32_t esz = F32 ? 4u : 2u;
    const uint32_t lane_off = (c.part * 64u + lane) * 16u + ((c.flag + rnd) & 1u) * sb;
    auto slice_len = [&](uint32_t s) -> uint32_t {
        const uint32_t lo = s * L;
        return lo >= a.n ? 0u : (a.n - lo < L ? a.n - lo : L);
    };
    // inbox offsets: receiver-major [recv][send]
    auto box = [&](uint32_t recv, uint32_t send) { return lane_off + (recv * N + send) * 2u * sb; };
    auto peer = [&](int j) { return wave + (uint32_t)(SENT_WAVES * j); };
    const bool act = e < slice_len(q);
    // ---- push my parts of this wave's slices
    u32x4 X[PW];
    uint32_t push = 0;
    // loads of this wave's parts, and below the polls, are issued by every
    // lane (nothing to move: at OFF_NONE), so they go out in one run instead
    // of each waiting behind a branch (16 ranks x 57344: 6.11 -> 5.68 us)
#pragma unroll
    for (int j = 0; j < PW; ++j) {
        const bool pj = peer(j) < N && peer(j) != q && e < slice_len(peer(j));
        X[j] = ld16<CP_PLAIN>(inq, pj ? (peer(j) * L + e) * 2u : OFF_NONE);
        if (pj)
            push |= 1u << j;
    }
    if (wave == 0u && act)
        stage[q][lane] = ld16<CP_PLAIN>(inq, (q * L + e) * 2u);
#pragma unroll
    for (int j = 0; j < PW; ++j)
        if ((push >> j) & 1u)
            st16<Pol<LOCAL>::ST>(X[j], rsr, box(peer(j), q));
    wait_stores();                  // receive only after the pushes are acknowledged
    u32x4 A0[PW], A1[PW], V[PW];
    uint32_t pend = 0;
    auto issue = [&](u32x4 *A, __amdgpu_buffer_rsrc_t reg) {
#pragma unroll
        for (int j = 0; j < PW; ++j)
            A[j] = ld16<Pol<LOCAL>::LD>(reg, ((pend >> j) & 1u) ? box(q, peer(j)) : OFF_NONE);
    };
    auto check = [&](const u32x4 *A) {
#pragma unroll
        for (int j = 0; j < PW; ++j)
            if ((pend >> j) & 1u)
                if (sent_ready(A[j])) {
                    pend &= ~(1u << j);
                    V[j] = A[j];
                }
    };
    auto receive = [&](__amdgpu_buffer_rsrc_t reg) {
        Watch w;
        w.begin(a.watchdog_ticks);
        issue(A0, reg);
        while (true) {
            compiler_fence();
            issue(A1, reg);
            check(A0);
            if (!wave_any(pend != 0u))
                break;
            if (w.expired(ctl, q, pend ? peer((int)first_bit(pend)) : 0u, c.call)) {
                *failed = 1u;                       // every wave still meets the barrier
                break;
            }
            compiler_fence();
            issue(A0, reg);
            check(A1);
            if (!wave_any(pend != 0u))
                break;
        }
    };
    // ---- receive my slice from this wave's peers, re-arm, stage
#pragma unroll
    for (int j = 0; j < PW; ++j)
        if (peer(j) < N && peer(j) != q && act)
            pend |= 1u << j;
    uint32_t mine = pend;
    receive(rsr);
    mark_once(c, c.t_sync);
#pragma unroll
    for (int j = 0; j < PW; ++j)
        if ((mine >> j) & 1u)
            stage[peer(j)][lane] = V[j];
    lds_barrier();                  // the tile only (the re-arm follows the reduce)
    if (*failed)
        return false;
    if (wave == 0u && act) {
        // every row of the tile at once (rows of absent ranks are not folded)
        u32x4 t[NMAX];
#pragma unroll
        for (int s = 0; s < NMAX; ++s)
            t[s] = stage[s][lane];
        Acc8 acc;
#pragma unroll
        for (int s = 0; s < NMAX; ++s)
            if ((uint32_t)s < N) {
                if (s == 0) acc.init(t[s]); else acc.add(t[s]);
            }
        if constexpr (F32) {
            // debug path: the owner writes its slice's accumulators to every copy
            for (uint32_t r = 0; r < N; ++r)
                store8<true>(oa, r * a.n + q * L + e, acc);
        } else {
            const u32x4 rv = acc.bf16();
            red[lane] = rv;
            st16<SENT_OUT>(rv, oa, (q * a.n + q * L + e) * esz);
        }
    }
    // re-arm the consumed reduce-scatter slots (resetRange); the round's
    // closing barrier waits for these stores before the next round's pushes
#pragma unroll
    for (int j = 0; j < PW; ++j)
        if ((mine >> j) & 1u)
            st16<Pol<LOCAL>::ST>(sentinel4(), rsr, box(q, peer(j)));
    if constexpr (F32) {                            // the debug path has no all-gather
        if (more)
            wait_stores();
        __syncthreads();
        return true;
    }
    __syncthreads();
    // ---- all-gather: push the reduced chunk to this wave's peers
    if (act) {
        const u32x4 rv = red[lane];
#pragma unroll
        for (int j = 0; j < PW; ++j)
            if (peer(j) < N && peer(j) != q)
                st16<Pol<LOCAL>::ST>(rv, agr, box(peer(j), q));
    }
    wait_stores();
    // ---- receive every other slice's reduced chunk from this wave's peers
    pend = 0;
#pragma unroll
    for (int j = 0; j < PW; ++j)
        if (peer(j) < N && peer(j) != q && e < slice_len(peer(j)))
            pend |= 1u << j;
    mine = pend;
    receive(agr);
#pragma unroll
    for (int j = 0; j < PW; ++j)
        if ((mine >> j) & 1u) {
            st16<SENT_OUT>(V[j], oa, (q * a.n + peer(j) * L + e) * esz);
            st16<Pol<LOCAL>::ST>(sentinel4(), agr, box(q, peer(j)));
        }
    // the round's re-arms (both inboxes) are performed before the next
    // round's pushes: a peer reuses a slot only after receiving such a push
    if (more)
        wait_stores();
    __syncthreads();                                // the tiles are reused next round
    return *failed == 0u;
}

template <int NMAX, bool F32, bool LOCAL, int HOOKS>
__global__ __launch_bounds__(512) void k_twoshot_sentinel(const Launch a)
{
    __shared__ u32x4 stage[NMAX][64];
    __shared__ u32x4 red[64];
    __shared__ uint32_t failed;
    Ctx0 c;
    begin<LOCAL, HOOKS>(a, c);
    const uint32_t N = a.n_ranks;
    const uint32_t G = a.slice >> 3;                // chunks per slice
    const uint32_t step = a.parts * 64u;
    const uint32_t rounds = (G + step - 1u) / step;
    if (threadIdx.x == 0)
        failed = 0u;
    load_seq(a, c);
    const Ctl ctl{a.ctl};
    const __amdgpu_buffer_rsrc_t inq = in_rsrc(a, c.rank);
    const __amdgpu_buffer_rsrc_t rsr = rsrc(a.srs, N * N * 2u * a.s2_stride);
    const __amdgpu_buffer_rsrc_t agr = rsrc(a.sag, N * N * 2u * a.s2_stride);
    const __amdgpu_buffer_rsrc_t oa = out_all(a, F32);
    uint32_t ch = c.part * 64u + (threadIdx.x & 63u);
    start_delay(a, c);
    // round 0 straight-line (see the one-shot LL kernel), later rounds looped
    if (!ts_round<NMAX, F32, LOCAL>(a, c, ctl, inq, rsr, agr, oa, ch, 0u, rounds > 1u, stage, red,
                                    &failed))
        return;
    for (uint32_t it = 1; it < rounds; ++it) {
        ch += step;
        if (!ts_round<NMAX, F32, LOCAL>(a, c, ctl, inq, rsr, agr, oa, ch, it, it + 1u < rounds,
                                        stage, red, &failed))
            return;
    }
    mark(c, c.t_data);
    finish(a, c);
}

// =========================================================== atomic lines
// The atomic two-phase algorithm of [EMC] ("四大核心机制", item 4: 128-byte
// blocks whose first 4 bytes are an atomic counter; every rank adds its data
// into the shared block with hardware atomics and bumps the counter; a block
// is complete when its counter reads N), on one GPU: binary32 atomic adds
// (performed where the device's atomics are, coherent for all workgroups)
// into lines of {counter, 31 x binary32} in a shared accumulator region.
//   phase 1 (reduce-scatter into the shared lines): each rank adds its 31
//     values of the line, waits until the adds are acknowledged, then adds 1
//     to the counter;
//   phase 2 (gather): each rank polls the counter until it reaches N, reads
//     the 31 sums and writes its output copy.
// The line cleans itself: after its read each rank adds 1 more, and the
// rank whose increment brings the counter to 2N (the last reader) zeroes
// the line.  So a line is zero again before the next call on that parity
// buffer can start (that call follows a call in which every rank completed
// this one), whatever protocols the calls in between used.
// The sums are taken in arrival order, so unlike every other kernel here the
// result is not the fixed-order fold: it is within (N-1) * 2^-24 * sum|x| of
// the exact sum before the bf16 rounding, and all N output copies agree.
// Lane layout: a wave holds two lines, a half-wave each; lane j of a half
// is the counter (j = 0) or element j-1 of the line.
constexpr uint32_t ATOM_ELEMS = (uint32_t)ATOM_LINE_ELEMS;     // binary32 sums per 128-byte line
constexpr uint32_t ATOM_LINE = 128;

template <int NMAX, bool F32, bool LOCAL, int HOOKS>
__global__ __launch_bounds__(256) void k_twoshot_atomic(const Launch a)
{
    Ctx0 c;
    begin<LOCAL, HOOKS>(a, c);
    const uint32_t N = a.n_ranks;
    const uint32_t lane = threadIdx.x & 63u, wave = threadIdx.x >> 6;
    const uint32_t half = lane >> 5, j = lane & 31u;
    const uint32_t lines = (a.n + ATOM_ELEMS - 1u) / ATOM_ELEMS;
    const uint32_t per_wg = (blockDim.x >> 6) * 2u;             // lines per workgroup round
    const uint32_t step = a.parts * per_wg;
    const __amdgpu_buffer_rsrc_t inr = in_rsrc(a, c.rank);
    const __amdgpu_buffer_rsrc_t o = out_rsrc(a, c.rank, F32);
    // accumulator lines [parity][line] x 128 B, zero between calls
    const __amdgpu_buffer_rsrc_t acc = rsrc(a.acc, 2u * a.acc_stride);
    const Ctl ctl{a.ctl};
    load_seq(a, c);
    start_delay(a, c);
    for (uint32_t l0 = c.part * per_wg; l0 < lines; l0 += step) {
        const uint32_t line = l0 + wave * 2u + half;
        const bool live = line < lines;
        const uint32_t e = line * ATOM_ELEMS + j - 1u;           // element of data lanes
        const bool data = live && j != 0u && e < a.n;
        const uint32_t base = c.par * a.acc_stride + line * ATOM_LINE;
        // phase 1: add this rank's values, then count this rank in
        if (data) {
            const uint32_t w = ld4<CP_PLAIN>(inr, (e & ~1u) * 2u);
            const float v = (e & 1u) ? hi_f(w) : lo_f(w);
            (void)__builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(v, acc, base + 4u * j, 0, 0);
        }
        wait_stores();                                          // the adds are performed
        if (live && j == 0u)
            (void)__builtin_amdgcn_raw_ptr_buffer_atomic_add_i32(1, acc, base, 0, 0);
        // phase 2: wait for all N ranks' adds (two polls in flight)
        bool pend = live && j == 0u;
        Watch w;
        w.begin(a.watchdog_ticks);
        uint32_t v0 = pend ? ld4<CP_DEV>(acc, base) : 0u, v1;
        bool ok = true;
        while (true) {
            compiler_fence();
            v1 = pend ? ld4<CP_DEV>(acc, base) : 0u;
            if (pend && v0 >= N)
                pend = false;
            if (!wave_any(pend))
                break;
            if (w.expired(ctl, c.rank, line, c.call)) {
                ok = false;
                break;
            }
            compiler_fence();
            v0 = pend ? ld4<CP_DEV>(acc, base) : 0u;
            if (pend && v1 >= N)
                pend = false;
            if (!wave_any(pend))
                break;
        }
        if (!ok)
            break;                      // status recorded; every wave still reaches finish()
        mark_once(c, c.t_sync);
        const uint32_t sb = data ? ld4<CP_DEV>(acc, base + 4u * j) : 0u;
        const float sum = __uint_as_float(sb);
        wait_stores();                                          // the read has returned
        // count this rank's read; the last reader zeroes the line
        uint32_t before = 0u;
        if (live && j == 0u)
            before = (uint32_t)__builtin_amdgcn_raw_ptr_buffer_atomic_add_i32(1, acc, base, 0, 0);
        const uint64_t last = __builtin_amdgcn_ballot_w64(live && j == 0u && before == 2u * N - 1u);
        if ((last >> (32u * half)) & 1u)
            st4<CP_DEV>(0u, acc, base + 4u * j);
        if (data) {
            if constexpr (F32)
                st4<CP_PLAIN>(__float_as_uint(sum), o, e * 4u);
            else
                __builtin_amdgcn_raw_buffer_store_b16(
                    (uint16_t)__builtin_bit_cast(uint16_t, (__bf16)sum), o, e * 2u, 0, CP_PLAIN);
        }
    }
    mark(c, c.t_data);
    finish(a, c);
}

// ============================================================ maintenance
// Closes a step of `calls` calls holding `rounds` rounds: advances the call
// count and the round sequence.  Round flags grow monotonically between
// clears; when the sequence passes SEQ_WRAP every flag word (LL units, LL128
// lines, arrival, barrier and completion flags, norm block sums) is cleared
// and the sequence restarts at 0, so a flag value left in memory can never
// match a later round.  (The host keeps a step below STEP_ROUNDS_MAX rounds,
// so no flag of a step reaches 2^32.)
__global__ __launch_bounds__(256) void k_step_end(uint32_t *ctl, uint32_t calls, uint32_t rounds,
                                                  char *ll, size_t ll_bytes, char *l128,
                                                  size_t l128_bytes, uint32_t *done,
                                                  uint32_t *stats, size_t stats_bytes)
{
    __shared__ uint32_t wrap;
    if (threadIdx.x == 0) {
        uint32_t s = __hip_atomic_load(ctl + CTL_SEQ, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        uint32_t next = s + rounds;
        wrap = (next > SEQ_WRAP || next < s) ? 1u : 0u;
    }
    __syncthreads();
    if (wrap) {
        uint32_t *w = (uint32_t *)ll;
        for (size_t i = threadIdx.x; i < ll_bytes / 4; i += blockDim.x) w[i] = 0u;
        w = (uint32_t *)l128;
        for (size_t i = threadIdx.x; i < l128_bytes / 4; i += blockDim.x) w[i] = 0u;
        for (size_t i = threadIdx.x; i < (size_t)MAX_RANKS * DONE_STRIDE; i += blockDim.x) done[i] = 0u;
        for (size_t i = threadIdx.x; i < stats_bytes / 4; i += blockDim.x) stats[i] = 0u;
        for (uint32_t i = threadIdx.x; i < (uint32_t)(CTL_WORDS - CTL_ARRIVE); i += blockDim.x)
            __hip_atomic_store(ctl + CTL_ARRIVE + i, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __threadfence();
    }
    // the arrival words restart with every step (their values are positions
    // in the step)
    for (uint32_t i = threadIdx.x; i < 32u * (uint32_t)XCDS; i += blockDim.x)
        __hip_atomic_store(ctl + CTL_ARRIVE + i, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t s = __hip_atomic_load(ctl + CTL_SEQ, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        uint32_t k = __hip_atomic_load(ctl + CTL_CALLS, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(ctl + CTL_SEQ, wrap ? 0u : s + rounds, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(ctl + CTL_CALLS, k + calls, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// Sets the round sequence to `seq` (a test hook: lets a test run steps
// across the sequence's restart without 2^28 steps before it).
__global__ __launch_bounds__(64) void k_set_seq(uint32_t *ctl, uint32_t seq)
{
    if (threadIdx.x == 0)
        __hip_atomic_store(ctl + CTL_SEQ, seq, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Fills `words` uint32 words with `value` (graph-capture safe replacement
// for a memset node).
__global__ __launch_bounds__(256) void k_fill(uint32_t *p, size_t words, uint32_t value)
{
    size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    size_t stride = (size_t)gridDim.x * blockDim.x;
    for (; i < words; i += stride)
        p[i] = value;
}

// Records the XCD of every workgroup: out[b] = XCC_ID of the workgroup with
// linear index b = x + gx (y + gy z) (grid gx x gy x gz).
__global__ __launch_bounds__(256) void k_xcc_map(uint32_t *out, uint32_t n, uint32_t gx, uint32_t gy)
{
    const uint32_t b = blockIdx.x + gx * (blockIdx.y + gy * blockIdx.z);
    if (threadIdx.x == 0 && b < n)
        out[b] = xcc_id();
}

// ------------------------------------------------------------ dispatch
// LL128 kernels by line groups per batch (1, 2, or 4 up to 8 ranks)
template <int NMAX, bool F32, bool LOCAL, int HOOKS>
static const void *pick_ll128(bool two, int gw)
{
    if (gw == 1)
        return two ? (const void *)k_twoshot_ll128<NMAX, F32, LOCAL, 1, HOOKS>
                   : (const void *)k_oneshot_ll128<NMAX, F32, LOCAL, 1, HOOKS>;
    if constexpr (NMAX > 8) {
        return two ? (const void *)k_twoshot_ll128<NMAX, F32, LOCAL, 2, HOOKS>
                   : (const void *)k_oneshot_ll128<NMAX, F32, LOCAL, 2, HOOKS>;
    } else {
        if (gw == 2)
            return two ? (const void *)k_twoshot_ll128<NMAX, F32, LOCAL, 2, HOOKS>
                       : (const void *)k_oneshot_ll128<NMAX, F32, LOCAL, 2, HOOKS>;
        return two ? (const void *)k_twoshot_ll128<NMAX, F32, LOCAL, 4, HOOKS>
                   : (const void *)k_oneshot_ll128<NMAX, F32, LOCAL, 4, HOOKS>;
    }
}

template <int NMAX, bool F32, bool LOCAL, int HOOKS>
static const void *pick(int kind, int gw)
{
    switch (kind) {
    case K_ONESHOT_LL: return (const void *)k_oneshot_ll<NMAX, F32, LOCAL, HOOKS>;
    case K_ONESHOT_SENTINEL: return (const void *)k_oneshot_sentinel<NMAX, F32, LOCAL, HOOKS>;
    case K_ONESHOT_DIRECT: return (const void *)k_oneshot_direct<NMAX, F32, LOCAL, HOOKS>;
    case K_ONESHOT_LL128: return pick_ll128<NMAX, F32, LOCAL, HOOKS>(false, gw);
    case K_TWOSHOT_LL128: return pick_ll128<NMAX, F32, LOCAL, HOOKS>(true, gw);
    case K_TWOSHOT_SENTINEL: return (const void *)k_twoshot_sentinel<NMAX, F32, LOCAL, HOOKS>;
    case K_TWOSHOT_DIRECT: return (const void *)k_twoshot_direct<NMAX, F32, LOCAL, HOOKS>;
    case K_ONESHOT_BARRIER: return (const void *)k_oneshot_barrier<NMAX, F32, LOCAL, HOOKS>;
    case K_TWOSHOT_BARRIER: return (const void *)k_twoshot_barrier<NMAX, F32, LOCAL, HOOKS>;
    case K_TWOSHOT_ATOMIC: return (const void *)k_twoshot_atomic<NMAX, F32, LOCAL, HOOKS>;
    case K_ONESHOT_LL_NORM:         // bf16 only
        return F32 ? nullptr : (const void *)k_oneshot_ll_norm<NMAX, LOCAL, HOOKS>;
    case K_ONESHOT_DIRECT_NORM:     // bf16 only
        return F32 ? nullptr : (const void *)k_oneshot_direct_norm<NMAX, LOCAL, HOOKS>;
    case K_ONESHOT_ROWS_NORM:       // bf16 only
        return F32 ? nullptr : (const void *)k_oneshot_rows_norm<NMAX, LOCAL, HOOKS>;
    default: return nullptr;
    }
}

template <int HOOKS>
static const void *pick_bf16(int kind, int n_ranks, bool local, int gw)
{
    if (n_ranks <= 8)
        return local ? pick<8, false, true, HOOKS>(kind, gw) : pick<8, false, false, HOOKS>(kind, gw);
    return local ? pick<16, false, true, HOOKS>(kind, gw) : pick<16, false, false, HOOKS>(kind, gw);
}

// The fp32 debug kernels always use device scope and always carry every hook.
const void *kernel_for(int kind, int n_ranks, bool f32, bool local, int gw, int hooks)
{
    if (f32)
        return n_ranks <= 8 ? pick<8, true, false, 2>(kind, gw) : pick<16, true, false, 2>(kind, gw);
    if (hooks <= 0)
        return pick_bf16<0>(kind, n_ranks, local, gw);
    if (hooks == 1)
        return pick_bf16<1>(kind, n_ranks, local, gw);
    return pick_bf16<2>(kind, n_ranks, local, gw);
}

// The hooks a launch record asks for (see begin).
static int hooks_of(const Launch &a)
{
    if (a.delays != nullptr || (a.ts != nullptr && a.ts_phases != 0u))
        return 2;
    return a.ts != nullptr ? 1 : 0;
}

// The grid of a launch record: (X, N, parts / X), X = 2^xshift.
static dim3 grid_of(const Launch &a)
{
    return dim3(1u << a.xshift, a.n_ranks, a.parts >> a.xshift);
}

hipError_t launch_ar(int kind, bool f32, bool local, int gw, const Launch &a, uint32_t threads,
                     hipStream_t stream)
{
    const void *fn = kernel_for(kind, (int)a.n_ranks, f32, local, gw, hooks_of(a));
    if (fn == nullptr || (a.parts & ((1u << a.xshift) - 1u)) != 0u)
        return hipErrorInvalidValue;
    if (kind == K_TWOSHOT_DIRECT || kind == K_ONESHOT_DIRECT) {
        uint32_t arr = a.rbase + 1u;        // the call's arrival value, first argument
        void *args2[] = {(void *)&arr, (void *)&a};
        return hipLaunchKernel(fn, grid_of(a), dim3(threads), args2, 0, stream);
    }
    void *args[] = {(void *)&a};
    return hipLaunchKernel(fn, grid_of(a), dim3(threads), args, 0, stream);
}

hipError_t launch_norm(int kind, bool local, const NormLaunch &L, uint32_t threads,
                       hipStream_t stream)
{
    if (kind != K_ONESHOT_LL_NORM && kind != K_ONESHOT_DIRECT_NORM && kind != K_ONESHOT_ROWS_NORM)
        return hipErrorInvalidValue;
    const void *fn = kernel_for(kind, (int)L.base.n_ranks, false, local, 0, hooks_of(L.base));
    if (fn == nullptr || (L.base.parts & ((1u << L.base.xshift) - 1u)) != 0u)
        return hipErrorInvalidValue;
    void *args[] = {(void *)&L};
    return hipLaunchKernel(fn, grid_of(L.base), dim3(threads), args, 0, stream);
}

hipError_t launch_xcc_map(uint32_t *out, uint32_t gx, uint32_t gy, uint32_t gz, uint32_t threads,
                          hipStream_t stream)
{
    hipLaunchKernelGGL(k_xcc_map, dim3(gx, gy, gz), dim3(threads), 0, stream, out, gx * gy * gz,
                       gx, gy);
    return hipGetLastError();
}

hipError_t launch_step_end(uint32_t *ctl, uint32_t calls, uint32_t rounds, char *ll,
                           size_t ll_bytes, char *l128, size_t l128_bytes, uint32_t *done,
                           uint32_t *stats, size_t stats_bytes, hipStream_t stream)
{
    hipLaunchKernelGGL(k_step_end, dim3(1), dim3(256), 0, stream, ctl, calls, rounds, ll, ll_bytes,
                       l128, l128_bytes, done, stats, stats_bytes);
    return hipGetLastError();
}

hipError_t launch_set_seq(uint32_t *ctl, uint32_t seq, hipStream_t stream)
{
    hipLaunchKernelGGL(k_set_seq, dim3(1), dim3(64), 0, stream, ctl, seq);
    return hipGetLastError();
}

hipError_t launch_fill(uint32_t *p, size_t words, uint32_t value, hipStream_t stream)
{
    if (words == 0)
        return hipSuccess;
    size_t blocks = (words + 255) / 256;
    if (blocks > 4096)
        blocks = 4096;
    hipLaunchKernelGGL(k_fill, dim3((unsigned)blocks), dim3(256), 0, stream, p, words, value);
    return hipGetLastError();
}

}  // namespace ar
