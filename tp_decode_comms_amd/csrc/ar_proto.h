// ar_proto.h -- device-side protocol layer of the barrier-free AllReduce (gfx950).
//
// The thread-level primitives of the "Every Microsecond Counts" write-up
// (page "微秒必争…", section "统一原语与API设计": send / recv / recvReduce /
// bcast / reset) become, on one MI355X whose "ranks" are workgroup sets:
//   publish  = device-coherent stores into a staging buffer (LL units, LL128
//              lines, or raw bf16 into a sentinel-armed inbox);
//   poll     = device-coherent loads repeated until in-band validity holds
//              (flag match, or no sentinel left), with a wave-wide vote and a
//              watchdog on the constant 100 MHz clock;
//   reduce   = an in-register binary32 left fold over ranks 0..N-1;
//   re-arm   = device-coherent stores of the sentinel over consumed slots.
//
// Memory access rules used throughout:
//   * every global access goes through a buffer resource whose record count
//     is the size of the buffer it names, so an index slip reads zeros and
//     drops stores instead of faulting;
//   * cross-workgroup traffic (staging, flags) uses the device-scope cache
//     policy (sc1): such loads do not hit stale lines in another XCD's L2
//     and such stores are written through to the device coherence point;
//   * a poll loop executes an empty asm statement with a memory clobber on
//     every iteration so that the compiler re-issues the loads.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ar {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// gfx950 buffer-instruction cache-policy bits
constexpr int CP_PLAIN = 0;
constexpr int CP_WG = 1;            // sc0: workgroup scope (coherent in the XCD's L2)
constexpr int CP_NT = 2;
constexpr int CP_DEV = 16;          // sc1: device-scope coherent

// Policies of the staging and flag traffic.  Device scope is coherent
// wherever the two sides run.  XCD-local scope (LOCAL) requires writer and
// reader on one XCD -- which the part-to-XCD mapping guarantees -- and then
// serves both from that XCD's L2: stores at workgroup scope, polls streaming
// at workgroup scope (they skip the CU's L1, so a repeated poll cannot hit a
// stale L1 line).  Measured on 8 ranks x 16 KiB: about 0.1-0.2 us less per call.
template <bool LOCAL> struct Pol {
    static constexpr int ST = LOCAL ? CP_WG : CP_DEV;
    static constexpr int LD = LOCAL ? (CP_NT | CP_WG) : CP_DEV;
};

constexpr int MAX_RANKS = 16;
constexpr uint32_t SENT_WORD = 0xFFFFFFFFu;   // two sentinel bf16 (0xFFFF)

// control block layout (uint32 words); each field on its own 128-byte line,
// except the two sequence words, which every launch reads together
constexpr int CTL_SEQ = 0;          // round-sequence base: flag of a step's first round - 1
constexpr int CTL_CALLS = 1;        // call-count base: number of calls before the step
constexpr int CTL_STATUS = 32;      // {code, rank, source, call}
// Workgroups are dispatched to the XCDs round-robin by workgroup index, so
// with `parts` a multiple of XCDS part p of every rank shares an XCD.
constexpr int XCDS = 8;
// arrival flag of rank r, copy x (read and written by workgroups of parts
// p = x mod XCDS) at word CTL_ARRIVE + 32*x + r: one 128-byte line per copy
constexpr int CTL_ARRIVE = 64;
// grid barrier of the barrier-ful baseline (one line per word): the arrival
// counters of the 8 workgroup groups, the group counter, and the XCDS
// copies of the top and of the bottom barrier's generation word
constexpr int CTL_BAR_GROUP = CTL_ARRIVE + 32 * XCDS;
constexpr int CTL_BAR_COUNT = CTL_BAR_GROUP + 32 * XCDS;
constexpr int CTL_BAR_TOP = CTL_BAR_COUNT + 32;
constexpr int CTL_BAR_BOTTOM = CTL_BAR_TOP + 32 * XCDS;
constexpr int CTL_WORDS = CTL_BAR_BOTTOM + 32 * XCDS;
static_assert(MAX_RANKS <= 32, "one arrival line holds every rank of a copy");
constexpr uint32_t STATUS_TIMEOUT = 6;
constexpr uint32_t DONE_STRIDE = 8192;    // completion-flag words per rank (>= workgroups per rank)
// Flags of a step stay below this value: the step-end kernel restarts the
// round sequence (clearing every flag word) before a step could reach it,
// and the host refuses a step of more than STEP_ROUNDS_MAX rounds, so no
// flag wraps around 2^32 between two clears.
constexpr uint32_t SEQ_WRAP = 0xF0000000u;
constexpr uint32_t STEP_ROUNDS_MAX = 0x08000000u;
// measurement records per wave: {start, first synchronisation satisfied,
// last data store issued, end}, constant-clock ticks
constexpr uint32_t TS_FIELDS = 4;

// LL128 line group: 8 lines of 128 B = one wave-wide 16 B access; 60 chunks
// of 8 elements carried as 56 full lanes + 8 half lanes (the lane at
// position 7 of each line keeps 8 B of payload and the line's 8 B flag).
constexpr uint32_t L128_ELEMS = 480;
constexpr uint32_t L128_BYTES = 1024;

struct Launch {
    const void *in[MAX_RANKS];    // rank inputs, bf16 [n]
    void *out;                    // [N][n] bf16 (or f32 for the debug path)
    char *ll;                     // LL units       [rank][parity] x ll_stride
    char *l128;                   // LL128 lines    [rank][parity] x l128_stride
    char *s1;                     // sentinel 1-shot [recv][send][parity] x s1_stride
    char *srs;                    // sentinel 2-shot RS inbox [recv][send][parity] x s2_stride
    char *sag;                    // sentinel 2-shot AG inbox [recv][send][parity] x s2_stride
    uint32_t *ctl;                // control block (CTL_WORDS)
    uint64_t *ts;                 // timestamps [slots][ts_stride][TS_FIELDS] or null
    const uint32_t *delays;       // start delays [rows][N] ns or null
    uint32_t *done;               // two-shot DIRECT completion flags (MAX_RANKS*DONE_STRIDE words)
    char *acc;                    // atomic accumulator lines [parity] x acc_stride, zero between calls
    uint32_t ll_stride, l128_stride, s1_stride, s2_stride, acc_stride;
    uint32_t n;                   // elements per rank
    uint32_t n_ranks;
    uint32_t epoch;               // call number within the step (1, 2, ...)
    uint32_t rbase;               // rounds of the step's earlier calls: round j's flag is
                                  // seq + rbase + 1 + j
    uint32_t parts;               // workgroups per rank
    uint32_t slice;               // two-shot slice length (multiple of 8)
    uint32_t watchdog_ticks;
    uint32_t xshift;              // log2 of parts per rank in a block (3, or 0): grid (2^xshift, N, parts >> xshift)
    uint32_t ts_slots;
    uint32_t ts_stride;           // records per slot (>= waves of the launch to be recorded)
    uint32_t ts_phases;           // nonzero: also record the two phase marks
    uint32_t delay_rows;
    uint32_t unit4;               // in-place one-shot: lanes take 4 elements (8 bytes), not 8
};

// The one-shot LL AllReduce with the residual add and RMS norm fused behind
// it.  base.out receives h [N][n]; y [N][n] the normalised rows.  Each
// 256-element block's sum of squares is published as {binary32 bits, flag}
// in stats[rank * stats_stride + block].
struct NormLaunch {
    Launch base;
    const void *res[MAX_RANKS];   // rank residuals, bf16 [n]
    const void *gamma;            // norm weight, bf16 [hidden], shared by all ranks
    void *y;                      // [N][n] bf16
    uint32_t *stats;              // [N][stats_stride] x 2 words
    uint32_t stats_stride;        // entries per rank (>= n / 256)
    uint32_t hidden;              // row length, a multiple of 256
    float eps;
};

// ---------------------------------------------------------------- buffers
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                             0x00020000);
}

// A byte offset past the end of every input and output descriptor (ar_init
// keeps them below 2^31 bytes): a raw buffer load at it returns zeros
// without a memory access, a store at it is dropped.  It lets a load or
// store that must be skipped still be issued unconditionally.  The poll
// loops also send the loads of lanes with nothing left to receive there;
// in a staging region of 2 GiB or more that offset can fall inside it,
// which is harmless for a load whose value is discarded (no store ever uses
// it on a staging descriptor).
constexpr uint32_t OFF_NONE = 0x80000000u;

template <int CP> __device__ __forceinline__ u32x4 ld16(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, CP);
}
template <int CP> __device__ __forceinline__ u32x2 ld8(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    return __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, CP);
}
template <int CP> __device__ __forceinline__ uint32_t ld4(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, CP);
}
template <int CP> __device__ __forceinline__ void st16(u32x4 v, __amdgpu_buffer_rsrc_t r, uint32_t off)
{
    __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, CP);
}
template <int CP> __device__ __forceinline__ void st8(u32x2 v, __amdgpu_buffer_rsrc_t r, uint32_t off)
{
    __builtin_amdgcn_raw_buffer_store_b64(v, r, off, 0, CP);
}
template <int CP> __device__ __forceinline__ void st4(uint32_t v, __amdgpu_buffer_rsrc_t r, uint32_t off)
{
    __builtin_amdgcn_raw_buffer_store_b32(v, r, off, 0, CP);
}

// Forces re-issue of loads inside a poll loop (no instruction is emitted).
__device__ __forceinline__ void compiler_fence() { asm volatile("" ::: "memory"); }

// Waits until this wave's earlier vector memory operations have completed:
// loads have returned and stores have been acknowledged.  For stores issued
// with the device-scope policy the acknowledgement means the data is at the
// device coherence point, so a flag stored afterwards is never seen before
// the payload.  Emitted through the builtin (s_waitcnt vmcnt(0), other
// counters untouched) so that the compiler's own wait insertion knows the
// counter is drained.
__device__ __forceinline__ void wait_stores()
{
    __builtin_amdgcn_s_waitcnt(0x0F70);
    compiler_fence();
}

// Workgroup barrier for exchanges through LDS only: waits for this wave's
// LDS operations (lgkmcnt(0); vector memory counters untouched), then
// s_barrier.  __syncthreads() also waits for every outstanding vector
// memory operation, which after a poll loop means the poll still in flight
// -- a round trip nobody needs when the barrier only orders the LDS tile.
// The compiler fences keep the LDS accesses on their side of it.
__device__ __forceinline__ void lds_barrier()
{
    compiler_fence();
    __builtin_amdgcn_s_waitcnt(0xC07F);
    __builtin_amdgcn_s_barrier();
    compiler_fence();
}

__device__ __forceinline__ uint64_t clock100() { return __builtin_amdgcn_s_memrealtime(); }

// index of the XCD this wave runs on (hardware register XCC_ID, bits 3:0)
__device__ __forceinline__ uint32_t xcc_id()
{
    return (uint32_t)__builtin_amdgcn_s_getreg((3 << 11) | (0 << 6) | 20) & 15u;
}

__device__ __forceinline__ bool wave_any(bool p)
{
    return __builtin_amdgcn_ballot_w64(p) != 0;
}

// ---------------------------------------------------------------- numerics
// bf16 pattern -> binary32 (exact widening: the pattern is the upper half).
__device__ __forceinline__ float lo_f(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_f(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// binary32 pair -> packed bf16 pair, round to nearest even (hardware
// v_cvt_pk_bf16_f32 on gfx950, reached through the bfloat16 conversion).
__device__ __forceinline__ uint32_t pack_bf16(float a, float b)
{
    __bf16 x = (__bf16)a;
    __bf16 y = (__bf16)b;
    return (uint32_t)__builtin_bit_cast(uint16_t, x) |
           ((uint32_t)__builtin_bit_cast(uint16_t, y) << 16);
}

// 4-element accumulator (one 8-byte lane chunk).
struct Acc4 {
    float v[4];
    __device__ __forceinline__ void init(uint32_t w0, uint32_t w1)
    {
        v[0] = lo_f(w0); v[1] = hi_f(w0); v[2] = lo_f(w1); v[3] = hi_f(w1);
    }
    __device__ __forceinline__ void add(uint32_t w0, uint32_t w1)
    {
        v[0] += lo_f(w0); v[1] += hi_f(w0); v[2] += lo_f(w1); v[3] += hi_f(w1);
    }
};

// 8-element accumulator.  init() starts from rank 0's values; add() is one
// binary32 addition per element, in the order the caller invokes it.
struct Acc8 {
    float v[8];
    __device__ __forceinline__ void init(u32x4 w)
    {
        v[0] = lo_f(w.x); v[1] = hi_f(w.x); v[2] = lo_f(w.y); v[3] = hi_f(w.y);
        v[4] = lo_f(w.z); v[5] = hi_f(w.z); v[6] = lo_f(w.w); v[7] = hi_f(w.w);
    }
    __device__ __forceinline__ void add(u32x4 w)
    {
        v[0] += lo_f(w.x); v[1] += hi_f(w.x); v[2] += lo_f(w.y); v[3] += hi_f(w.y);
        v[4] += lo_f(w.z); v[5] += hi_f(w.z); v[6] += lo_f(w.w); v[7] += hi_f(w.w);
    }
    __device__ __forceinline__ u32x4 bf16() const
    {
        u32x4 r;
        r.x = pack_bf16(v[0], v[1]); r.y = pack_bf16(v[2], v[3]);
        r.z = pack_bf16(v[4], v[5]); r.w = pack_bf16(v[6], v[7]);
        return r;
    }
};

// ---------------------------------------------------------------- LL units
// One 16-byte LL store carries two 8-byte units {payload word, flag}.  Each
// unit validates itself, so a 16-byte access that tears at 8-byte
// granularity is harmless.
__device__ __forceinline__ u32x4 ll_pack(uint32_t w0, uint32_t w1, uint32_t flag)
{
    u32x4 r; r.x = w0; r.y = flag; r.z = w1; r.w = flag; return r;
}
__device__ __forceinline__ bool ll_ready(u32x4 u, uint32_t flag)
{
    return u.y == flag && u.w == flag;
}

// ---------------------------------------------------------------- sentinel
__device__ __forceinline__ bool no_sentinel(uint32_t w)
{
    return (w & 0xFFFFu) != 0xFFFFu && (w >> 16) != 0xFFFFu;
}
__device__ __forceinline__ bool sent_ready(u32x4 v)
{
    return no_sentinel(v.x) && no_sentinel(v.y) && no_sentinel(v.z) && no_sentinel(v.w);
}
__device__ __forceinline__ u32x4 sentinel4()
{
    u32x4 r; r.x = SENT_WORD; r.y = SENT_WORD; r.z = SENT_WORD; r.w = SENT_WORD; return r;
}

// ---------------------------------------------------------------- LL128 lanes
// Lane l of a wave holds, for one line group:
//   l % 8 != 7: chunk c = 7*(l/8) + l%8, elements [8c, 8c+8)  -> 16 B payload
//   l % 8 == 7: half chunk h = l/8, elements [448+4h, 448+4h+4) -> 8 B payload
//               followed by the line's 8 B flag.
struct L128Lane {
    uint32_t elem;     // first element of this lane within the group
    bool half;         // flag lane (4 elements)
};
__device__ __forceinline__ L128Lane l128_lane(uint32_t lane)
{
    L128Lane r;
    uint32_t line = lane >> 3, j = lane & 7u;
    r.half = (j == 7u);
    r.elem = r.half ? (448u + 4u * line) : 8u * (7u * line + j);
    return r;
}

// ---------------------------------------------------------------- control
struct Ctl {
    uint32_t *p;
    __device__ __forceinline__ uint32_t status() const
    {
        return __hip_atomic_load(p + CTL_STATUS, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __device__ __forceinline__ void fail(uint32_t rank, uint32_t src, uint32_t flag,
                                         uint32_t code = STATUS_TIMEOUT) const
    {
        uint32_t expected = 0;
        if (__hip_atomic_compare_exchange_strong(p + CTL_STATUS, &expected, code,
                                                 __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT)) {
            __hip_atomic_store(p + CTL_STATUS + 1, rank, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(p + CTL_STATUS + 2, src, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(p + CTL_STATUS + 3, flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
};

// Poll-loop bookkeeping: watchdog on the 100 MHz clock, and an early exit
// once any workgroup has recorded a failure.  Wave-uniform.
// LAZY: the budget runs from the first poll that finds nothing (the clock
// is read then, not before the first poll: a clock read is a scalar-memory
// instruction that the next LDS wait also waits for; 8 x 512 KiB LL128
// one-shot 7.83 -> 7.49 us, 16 ranks x 57344 sentinel two-shot 5.42 ->
// 5.30).  The one-shot LL receive keeps the clock read before its first
// poll (the lazy form measured 0.015 us slower there).
template <bool LAZY>
struct WatchT {
    uint64_t start;
    uint32_t budget;
    uint32_t iter;
    __device__ __forceinline__ void begin(uint32_t ticks)
    {
        start = LAZY ? 0u : clock100();
        budget = ticks;
        iter = 0;
    }
    // true -> give up (status already recorded by someone, or recorded now)
    __device__ __forceinline__ bool expired(const Ctl &c, uint32_t rank, uint32_t src, uint32_t flag)
    {
        ++iter;
        if ((iter & 63u) == 0u && c.status() != 0u)
            return true;
        const uint64_t now = clock100();
        if constexpr (LAZY) {
            if (start == 0u) {
                start = now;
                return false;
            }
        }
        if (now - start > budget) {
            c.fail(rank, src, flag);
            return true;
        }
        return false;
    }
};
using Watch = WatchT<true>;

// lowest set bit index of a non-zero mask
__device__ __forceinline__ uint32_t first_bit(uint32_t m) { return (uint32_t)__builtin_ctz(m); }

}  // namespace ar
