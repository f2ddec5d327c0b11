// ar_kernels.hip -- gfx950 kernels of the barrier-free fixed-order AllReduce.
//
// One launch = one AllReduce call for all N emulated ranks.  Workgroup b
// belongs to rank b % N and covers part b / N of that rank's work, so with
// the hardware's round-robin workgroup-to-XCD dispatch every rank of an
// 8-rank call lives on one XCD and every exchange between ranks crosses XCD
// L2 caches, as exchanges between GPUs cross the fabric.  Workgroups of one
// part index depend only on each other, and the host never launches more
// workgroups than the device holds at once, so every poll has a resident
// producer.
//
// Algorithms ("Every Microsecond Counts" write-up, page "微秒必争…", section
// "统一原语与API设计" and its table of variants):
//   one-shot: read local value, publish, receive-and-reduce all N, write;
//   two-shot: reduce-scatter (rank q reduces slice q) then all-gather.
// Protocols (same page, section "四大核心机制"): LL units, sentinel inboxes,
// parity double buffering, LL128-style lines; plus DIRECT, which reads peers'
// inputs in place once their per-call arrival flag is up.
//
// Summation order is the global rank order 0..N-1 for every element on
// every rank and in both algorithms, so all variants give identical bits.
#include "ar_proto.h"
#include "ar_kernels.h"

namespace ar {

// ------------------------------------------------------------------ common
struct Ctx0 {
    uint32_t rank, part, flag, par;
    uint64_t t0;
};

__device__ __forceinline__ uint32_t load_seq(const Launch &a)
{
    return __hip_atomic_load(a.ctl + CTL_SEQ, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void start_delay(const Launch &a, const Ctx0 &c)
{
    if (a.delays == nullptr)
        return;
    __amdgpu_buffer_rsrc_t d = rsrc(a.delays, a.delay_rows * a.n_ranks * 4u);
    uint32_t row = (c.flag - 1u) % a.delay_rows;
    uint32_t ns = ld4<CP_PLAIN>(d, (row * a.n_ranks + c.rank) * 4u);
    uint64_t ticks = ns / 10u;
    if (ticks > 1000000u)                 // at most 10 ms per call
        ticks = 1000000u;
    while (clock100() - c.t0 < ticks)
        __builtin_amdgcn_s_sleep(1);
}

__device__ __forceinline__ void finish(const Launch &a, const Ctx0 &c)
{
    if (a.ts == nullptr)
        return;
    wait_stores();
    __syncthreads();
    if (threadIdx.x == 0) {
        uint64_t t1 = clock100();
        uint32_t slot = (c.flag - 1u) % a.ts_slots;
        __hip_atomic_fetch_min(a.ts + 2 * slot, c.t0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_fetch_max(a.ts + 2 * slot + 1, t1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

template <bool F32>
__device__ __forceinline__ void store_out8(const Launch &a, uint32_t rank, uint32_t elem,
                                           const Acc8 &acc)
{
    // elem is a multiple of 8 inside [0, n)
    if constexpr (F32) {
        char *base = (char *)a.out + (size_t)rank * a.n * 4u;
        __amdgpu_buffer_rsrc_t o = rsrc(base, a.n * 4u);
        u32x4 lo, hi;
        lo.x = __float_as_uint(acc.v[0]); lo.y = __float_as_uint(acc.v[1]);
        lo.z = __float_as_uint(acc.v[2]); lo.w = __float_as_uint(acc.v[3]);
        hi.x = __float_as_uint(acc.v[4]); hi.y = __float_as_uint(acc.v[5]);
        hi.z = __float_as_uint(acc.v[6]); hi.w = __float_as_uint(acc.v[7]);
        st16<CP_PLAIN>(lo, o, elem * 4u);
        st16<CP_PLAIN>(hi, o, elem * 4u + 16u);
    } else {
        char *base = (char *)a.out + (size_t)rank * a.n * 2u;
        __amdgpu_buffer_rsrc_t o = rsrc(base, a.n * 2u);
        st16<CP_PLAIN>(acc.bf16(), o, elem * 2u);
    }
}

// 4-element variant (LL128 flag lanes): values in acc.v[0..3]
template <bool F32>
__device__ __forceinline__ void store_out4(const Launch &a, uint32_t rank, uint32_t elem,
                                           const Acc8 &acc)
{
    if constexpr (F32) {
        char *base = (char *)a.out + (size_t)rank * a.n * 4u;
        __amdgpu_buffer_rsrc_t o = rsrc(base, a.n * 4u);
        u32x4 lo;
        lo.x = __float_as_uint(acc.v[0]); lo.y = __float_as_uint(acc.v[1]);
        lo.z = __float_as_uint(acc.v[2]); lo.w = __float_as_uint(acc.v[3]);
        st16<CP_PLAIN>(lo, o, elem * 4u);
    } else {
        char *base = (char *)a.out + (size_t)rank * a.n * 2u;
        __amdgpu_buffer_rsrc_t o = rsrc(base, a.n * 2u);
        u32x2 w; w.x = pack_bf16(acc.v[0], acc.v[1]); w.y = pack_bf16(acc.v[2], acc.v[3]);
        st8<CP_PLAIN>(w, o, elem * 2u);
    }
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t in_rsrc(const Launch &a, uint32_t r)
{
    return rsrc(a.in[r], a.n * 2u);
}

// ============================================================ one-shot LL
// Lane work unit: chunk c of 8 elements (16 B of input).  Rank r publishes
// chunk c as two 16-byte LL stores: elements 0..3 at byte 16c of the first
// half of its mailbox and elements 4..7 at byte 16c of the second half, so
// both the stores and every reader's loads are contiguous across a wave.
template <int NMAX, bool F32>
__global__ __launch_bounds__(256) void k_oneshot_ll(const Launch a)
{
    Ctx0 c;
    c.t0 = clock100();
    c.rank = blockIdx.x % a.n_ranks;
    c.part = blockIdx.x / a.n_ranks;
    const uint32_t N = a.n_ranks;
    const uint32_t G = a.n >> 3;                    // chunks per rank
    const uint32_t half = G * 16u;                  // byte offset of the second half
    const uint32_t mb_bytes = G * 32u;
    const uint32_t step = a.parts * blockDim.x;
    const uint32_t rounds = (G + step - 1u) / step;
    uint32_t seq = load_seq(a);
    c.flag = seq + a.epoch;
    c.par = a.epoch & 1u;
    const Ctl ctl{a.ctl};
    __amdgpu_buffer_rsrc_t mine = rsrc(a.ll + (size_t)(c.rank * 2u + c.par) * a.ll_stride, mb_bytes);
    __amdgpu_buffer_rsrc_t src[NMAX];
#pragma unroll
    for (int s = 0; s < NMAX; ++s)
        src[s] = rsrc(a.ll + (size_t)((uint32_t)s * 2u + c.par) * a.ll_stride, mb_bytes);
    const __amdgpu_buffer_rsrc_t inr = in_rsrc(a, c.rank);

    for (uint32_t it = 0; it < rounds; ++it) {
        const uint32_t ch = c.part * blockDim.x + threadIdx.x + it * step;
        const bool active = ch < G;
        u32x4 x = {0u, 0u, 0u, 0u};
        if (active)
            x = ld16<CP_PLAIN>(inr, ch * 16u);
        if (it == 0)
            start_delay(a, c);
        // publish (send/bcast): one copy, read by all N ranks
        if (active) {
            st16<CP_DEV>(ll_pack(x.x, x.y, c.flag), mine, ch * 16u);
            st16<CP_DEV>(ll_pack(x.z, x.w, c.flag), mine, half + ch * 16u);
        }
        // receive: poll every peer's units for this chunk
        u32x4 A[NMAX], B[NMAX];
        uint32_t pend = 0;
#pragma unroll
        for (int s = 0; s < NMAX; ++s) {
            if ((uint32_t)s < N && (uint32_t)s != c.rank && active) {
                A[s] = ld16<CP_DEV>(src[s], ch * 16u);
                B[s] = ld16<CP_DEV>(src[s], half + ch * 16u);
                pend |= 1u << s;
            }
        }
        Watch w;
        w.begin(a.watchdog_ticks);
        while (true) {
#pragma unroll
            for (int s = 0; s < NMAX; ++s)
                if ((pend >> s) & 1u)
                    if (ll_ready(A[s], c.flag) && ll_ready(B[s], c.flag))
                        pend &= ~(1u << s);
            if (!wave_any(pend != 0u))
                break;
            if (w.expired(ctl, c.rank, pend ? first_bit(pend) : 0u, c.flag))
                return;
            compiler_fence();
#pragma unroll
            for (int s = 0; s < NMAX; ++s) {
                if ((pend >> s) & 1u) {
                    A[s] = ld16<CP_DEV>(src[s], ch * 16u);
                    B[s] = ld16<CP_DEV>(src[s], half + ch * 16u);
                }
            }
        }
        // reduce in global rank order, own value from registers
        if (active) {
            Acc8 acc;
#pragma unroll
            for (int s = 0; s < NMAX; ++s) {
                if ((uint32_t)s < N) {
                    u32x4 v;
                    if ((uint32_t)s == c.rank) {
                        v = x;
                    } else {
                        v.x = A[s].x; v.y = A[s].z; v.z = B[s].x; v.w = B[s].z;
                    }
                    if (s == 0) acc.init(v); else acc.add(v);
                }
            }
            store_out8<F32>(a, c.rank, ch * 8u, acc);
        }
    }
    finish(a, c);
}

// ======================================================= one-shot sentinel
// Push model: rank q writes chunk c of its input into every peer's inbox
// [peer][q][parity]; each receiver polls its own inbox until no element is
// the sentinel, reduces, and re-arms the slots it consumed.  The receipt of
// a peer's call-k data proves the peer finished call k-1 (double buffering),
// so the re-arm of parity k&1 always lands before the peer's call k+2 write.
template <int NMAX, bool F32>
__global__ __launch_bounds__(256) void k_oneshot_sentinel(const Launch a)
{
    Ctx0 c;
    c.t0 = clock100();
    c.rank = blockIdx.x % a.n_ranks;
    c.part = blockIdx.x / a.n_ranks;
    const uint32_t N = a.n_ranks;
    const uint32_t G = a.n >> 3;
    const uint32_t bytes = a.n * 2u;
    const uint32_t step = a.parts * blockDim.x;
    const uint32_t rounds = (G + step - 1u) / step;
    uint32_t seq = load_seq(a);
    c.flag = seq + a.epoch;
    c.par = a.epoch & 1u;
    const Ctl ctl{a.ctl};
    const __amdgpu_buffer_rsrc_t inr = in_rsrc(a, c.rank);
    // inbox(recv, send) = s1 + ((recv*N + send)*2 + par) * stride
    auto inbox = [&](uint32_t recv, uint32_t send) {
        return rsrc(a.s1 + (size_t)((recv * N + send) * 2u + c.par) * a.s1_stride, bytes);
    };

    for (uint32_t it = 0; it < rounds; ++it) {
        const uint32_t ch = c.part * blockDim.x + threadIdx.x + it * step;
        const bool active = ch < G;
        u32x4 x = {0u, 0u, 0u, 0u};
        if (active)
            x = ld16<CP_PLAIN>(inr, ch * 16u);
        if (it == 0)
            start_delay(a, c);
        if (active) {
#pragma unroll
            for (int s = 0; s < NMAX; ++s)
                if ((uint32_t)s < N && (uint32_t)s != c.rank)
                    st16<CP_DEV>(x, inbox((uint32_t)s, c.rank), ch * 16u);
        }
        u32x4 V[NMAX];
        uint32_t pend = 0;
#pragma unroll
        for (int s = 0; s < NMAX; ++s) {
            if ((uint32_t)s < N && (uint32_t)s != c.rank && active) {
                V[s] = ld16<CP_DEV>(inbox(c.rank, (uint32_t)s), ch * 16u);
                pend |= 1u << s;
            }
        }
        Watch w;
        w.begin(a.watchdog_ticks);
        while (true) {
#pragma unroll
            for (int s = 0; s < NMAX; ++s)
                if ((pend >> s) & 1u)
                    if (sent_ready(V[s]))
                        pend &= ~(1u << s);
            if (!wave_any(pend != 0u))
                break;
            if (w.expired(ctl, c.rank, pend ? first_bit(pend) : 0u, c.flag))
                return;
            compiler_fence();
#pragma unroll
            for (int s = 0; s < NMAX; ++s)
                if ((pend >> s) & 1u)
                    V[s] = ld16<CP_DEV>(inbox(c.rank, (uint32_t)s), ch * 16u);
        }
        if (active) {
            Acc8 acc;
#pragma unroll
            for (int s = 0; s < NMAX; ++s) {
                if ((uint32_t)s < N) {
                    u32x4 v = ((uint32_t)s == c.rank) ? x : V[s];
                    if (s == 0) acc.init(v); else acc.add(v);
                }
            }
            // re-arm what was consumed (resetRange), then write the result
#pragma unroll
            for (int s = 0; s < NMAX; ++s)
                if ((uint32_t)s < N && (uint32_t)s != c.rank)
                    st16<CP_DEV>(sentinel4(), inbox(c.rank, (uint32_t)s), ch * 16u);
            store_out8<F32>(a, c.rank, ch * 8u, acc);
        }
    }
    finish(a, c);
}

// ========================================================= one-shot DIRECT
// Every workgroup of rank r raises r's arrival flag for this call; a reader
// of rank s's input waits until s's arrival flag has reached the call's flag
// and then reads in[s] in place.  Meant for messages too large for staging
// copies; the input of call k must stay unchanged until call k completes on
// every rank (the application-level A/B double buffering of the SiFAR page,
// "SiFAR：无同步All-Reduce技术突破低延迟LLM推理瓶颈", technique one).
__device__ __forceinline__ bool wait_arrivals(const Launch &a, const Ctx0 &c, const Ctl &ctl)
{
    const uint32_t lane = threadIdx.x & 63u;
    bool need = lane < a.n_ranks;
    uint32_t off = (CTL_ARRIVE + 32u * lane) * 4u;
    __amdgpu_buffer_rsrc_t r = rsrc(a.ctl, CTL_WORDS * 4u);
    Watch w;
    w.begin(a.watchdog_ticks);
    while (true) {
        if (need) {
            uint32_t v = ld4<CP_DEV>(r, off);
            if ((int32_t)(v - c.flag) >= 0)
                need = false;
        }
        if (!wave_any(need))
            return true;
        if (w.expired(ctl, c.rank, lane, c.flag))
            return false;
        compiler_fence();
    }
}

__device__ __forceinline__ void raise_arrival(const Launch &a, const Ctx0 &c)
{
    if (threadIdx.x == 0) {
        __amdgpu_buffer_rsrc_t r = rsrc(a.ctl, CTL_WORDS * 4u);
        st4<CP_DEV>(c.flag, r, (CTL_ARRIVE + 32u * c.rank) * 4u);
    }
}

template <int NMAX, bool F32>
__global__ __launch_bounds__(256) void k_oneshot_direct(const Launch a)
{
    Ctx0 c;
    c.t0 = clock100();
    c.rank = blockIdx.x % a.n_ranks;
    c.part = blockIdx.x / a.n_ranks;
    const uint32_t N = a.n_ranks;
    const uint32_t G = a.n >> 3;
    const uint32_t step = a.parts * blockDim.x;
    const uint32_t rounds = (G + step - 1u) / step;
    uint32_t seq = load_seq(a);
    c.flag = seq + a.epoch;
    c.par = a.epoch & 1u;
    const Ctl ctl{a.ctl};
    start_delay(a, c);
    raise_arrival(a, c);
    if (!wait_arrivals(a, c, ctl))
        return;
    __amdgpu_buffer_rsrc_t src[NMAX];
#pragma unroll
    for (int s = 0; s < NMAX; ++s)
        src[s] = in_rsrc(a, (uint32_t)s < N ? (uint32_t)s : 0u);
    for (uint32_t it = 0; it < rounds; ++it) {
        const uint32_t ch = c.part * blockDim.x + threadIdx.x + it * step;
        if (ch >= G)
            continue;
        u32x4 V[NMAX];
#pragma unroll
        for (int s = 0; s < NMAX; ++s)
            if ((uint32_t)s < N)
                V[s] = ld16<CP_PLAIN>(src[s], ch * 16u);
        Acc8 acc;
#pragma unroll
        for (int s = 0; s < NMAX; ++s)
            if ((uint32_t)s < N) {
                if (s == 0) acc.init(V[s]); else acc.add(V[s]);
            }
        store_out8<F32>(a, c.rank, ch * 8u, acc);
    }
    finish(a, c);
}

// ============================================================ LL128 lines
// Writes one lane's share of a line group: payload first; after every
// payload store of the wave has been acknowledged at the device coherence
// point, the flag lanes store the line flags.
__device__ __forceinline__ void l128_publish(__amdgpu_buffer_rsrc_t dst, uint32_t goff,
                                             uint32_t lane, const L128Lane &ln, u32x4 payload,
                                             uint32_t flag)
{
    const uint32_t off = goff + lane * 16u;
    if (ln.half) {
        u32x2 p; p.x = payload.x; p.y = payload.y;
        st8<CP_DEV>(p, dst, off);
    } else {
        st16<CP_DEV>(payload, dst, off);
    }
    wait_stores();
    if (ln.half) {
        u32x2 f; f.x = flag; f.y = ~flag;
        st8<CP_DEV>(f, dst, off + 8u);
    }
}

__device__ __forceinline__ bool l128_flag_ok(u32x2 f, uint32_t flag)
{
    return f.x == flag && f.y == ~flag;
}

// Reads one line group of the N sources: flag lanes poll their line flags,
// the wave votes, then every lane loads its payload.  lim[s] is the number
// of valid elements of source s in the group index space; a line is polled
// when any of its elements is valid.  Returns false on watchdog expiry.
// `skip` names a source the caller already holds (or NMAX for none).
template <int NMAX>
__device__ __forceinline__ bool l128_receive(const __amdgpu_buffer_rsrc_t *src, uint32_t N,
                                             uint32_t skip, uint32_t g, uint32_t lane,
                                             const L128Lane &ln, const uint32_t *lim,
                                             uint32_t flag, const Ctl &ctl, uint32_t rank,
                                             uint32_t budget, u32x4 *V)
{
    const uint32_t goff = g * L128_BYTES;
    const uint32_t off = goff + lane * 16u;
    const uint32_t e = g * L128_ELEMS + ln.elem;
    const uint32_t line_first = g * L128_ELEMS + 56u * (lane >> 3);
    uint32_t pend = 0;
    u32x2 F[NMAX];
#pragma unroll
    for (int s = 0; s < NMAX; ++s) {
        if ((uint32_t)s < N && (uint32_t)s != skip && ln.half && line_first < lim[s]) {
            F[s] = ld8<CP_DEV>(src[s], off + 8u);
            pend |= 1u << s;
        }
    }
    Watch w;
    w.begin(budget);
    while (true) {
#pragma unroll
        for (int s = 0; s < NMAX; ++s)
            if ((pend >> s) & 1u)
                if (l128_flag_ok(F[s], flag))
                    pend &= ~(1u << s);
        if (!wave_any(pend != 0u))
            break;
        if (w.expired(ctl, rank, pend ? first_bit(pend) : 0u, flag))
            return false;
        compiler_fence();
#pragma unroll
        for (int s = 0; s < NMAX; ++s)
            if ((pend >> s) & 1u)
                F[s] = ld8<CP_DEV>(src[s], off + 8u);
    }
    // every needed line of the group is complete: read the payloads
    compiler_fence();
#pragma unroll
    for (int s = 0; s < NMAX; ++s) {
        if ((uint32_t)s < N && (uint32_t)s != skip && e < lim[s]) {
            if (ln.half) {
                u32x2 p = ld8<CP_DEV>(src[s], off);
                V[s].x = p.x; V[s].y = p.y; V[s].z = 0u; V[s].w = 0u;
            } else {
                V[s] = ld16<CP_DEV>(src[s], off);
            }
        }
    }
    return true;
}

// reads 8 (or 4) elements of a bf16 buffer at element `e`
__device__ __forceinline__ u32x4 ld_elems(__amdgpu_buffer_rsrc_t r, uint32_t e, bool half)
{
    if (half) {
        u32x2 p = ld8<CP_PLAIN>(r, e * 2u);
        u32x4 v; v.x = p.x; v.y = p.y; v.z = 0u; v.w = 0u;
        return v;
    }
    return ld16<CP_PLAIN>(r, e * 2u);
}

template <bool F32>
__device__ __forceinline__ void store_lane(const Launch &a, uint32_t rank, uint32_t e, bool half,
                                           const Acc8 &acc)
{
    if (half) store_out4<F32>(a, rank, e, acc); else store_out8<F32>(a, rank, e, acc);
}

// ====================================================== one-shot LL128
// Rank r publishes its whole input as line groups (480 elements each); each
// wave owns a set of groups, publishes all of them, then receives and
// reduces the same groups from every rank.
template <int NMAX, bool F32>
__global__ __launch_bounds__(256) void k_oneshot_ll128(const Launch a)
{
    Ctx0 c;
    c.t0 = clock100();
    c.rank = blockIdx.x % a.n_ranks;
    c.part = blockIdx.x / a.n_ranks;
    const uint32_t N = a.n_ranks;
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t wave = threadIdx.x >> 6;
    const uint32_t waves = blockDim.x >> 6;
    const uint32_t groups = (a.n + L128_ELEMS - 1u) / L128_ELEMS;
    const uint32_t gstep = a.parts * waves;
    const uint32_t g0 = c.part * waves + wave;
    const uint32_t mb_bytes = groups * L128_BYTES;
    uint32_t seq = load_seq(a);
    c.flag = seq + a.epoch;
    c.par = a.epoch & 1u;
    const Ctl ctl{a.ctl};
    const L128Lane ln = l128_lane(lane);
    const __amdgpu_buffer_rsrc_t inr = in_rsrc(a, c.rank);
    __amdgpu_buffer_rsrc_t src[NMAX];
#pragma unroll
    for (int s = 0; s < NMAX; ++s)
        src[s] = rsrc(a.l128 + (size_t)((uint32_t)s * 2u + c.par) * a.l128_stride, mb_bytes);

    bool first = true;
    for (uint32_t g = g0; g < groups; g += gstep) {
        const uint32_t e = g * L128_ELEMS + ln.elem;
        const bool active = e < a.n;
        u32x4 x = {0u, 0u, 0u, 0u};
        if (active)
            x = ld_elems(inr, e, ln.half);
        if (first) { start_delay(a, c); first = false; }
        l128_publish(src[c.rank], g * L128_BYTES, lane, ln, x, c.flag);
    }
    if (first)
        start_delay(a, c);
    for (uint32_t g = g0; g < groups; g += gstep) {
        const uint32_t e = g * L128_ELEMS + ln.elem;
        const bool active = e < a.n;
        u32x4 V[NMAX];
        uint32_t lim[NMAX];
#pragma unroll
        for (int s = 0; s < NMAX; ++s) lim[s] = a.n;
        if (!l128_receive<NMAX>(src, N, c.rank, g, lane, ln, lim, c.flag, ctl, c.rank,
                                a.watchdog_ticks, V))
            return;
        if (active) {
            u32x4 x = ld_elems(inr, e, ln.half);
            Acc8 acc;
#pragma unroll
            for (int s = 0; s < NMAX; ++s) {
                if ((uint32_t)s < N) {
                    u32x4 v = ((uint32_t)s == c.rank) ? x : V[s];
                    if (s == 0) acc.init(v); else acc.add(v);
                }
            }
            store_lane<F32>(a, c.rank, e, ln.half, acc);
        }
    }
    finish(a, c);
}

// ====================================================== two-shot LL128
// Reduce-scatter: rank q reduces slice q (elements [q*L, q*L + Lq)) reading
// every rank's input in place after its arrival flag, and publishes the
// bf16 result as line groups.  All-gather: rank q receives every slice's
// groups and writes them to out[q].  A wave owns the same group indices in
// both phases, so its own slice's result stays in registers.
template <int NMAX, bool F32>
__global__ __launch_bounds__(256) void k_twoshot_ll128(const Launch a)
{
    Ctx0 c;
    c.t0 = clock100();
    c.rank = blockIdx.x % a.n_ranks;
    c.part = blockIdx.x / a.n_ranks;
    const uint32_t N = a.n_ranks;
    const uint32_t q = c.rank;
    const uint32_t L = a.slice;
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t wave = threadIdx.x >> 6;
    const uint32_t waves = blockDim.x >> 6;
    const uint32_t groups = (L + L128_ELEMS - 1u) / L128_ELEMS;
    const uint32_t gstep = a.parts * waves;
    const uint32_t g0 = c.part * waves + wave;
    const uint32_t mb_bytes = groups * L128_BYTES;
    uint32_t seq = load_seq(a);
    c.flag = seq + a.epoch;
    c.par = a.epoch & 1u;
    const Ctl ctl{a.ctl};
    const L128Lane ln = l128_lane(lane);
    auto slice_len = [&](uint32_t s) -> uint32_t {
        uint32_t lo = s * L;
        return lo >= a.n ? 0u : (a.n - lo < L ? a.n - lo : L);
    };
    start_delay(a, c);
    raise_arrival(a, c);
    if (!wait_arrivals(a, c, ctl))
        return;
    __amdgpu_buffer_rsrc_t inp[NMAX], stg[NMAX];
#pragma unroll
    for (int s = 0; s < NMAX; ++s) {
        uint32_t ss = (uint32_t)s < N ? (uint32_t)s : 0u;
        inp[s] = in_rsrc(a, ss);
        stg[s] = rsrc(a.l128 + (size_t)(ss * 2u + c.par) * a.l128_stride, mb_bytes);
    }
    const uint32_t Lq = slice_len(q);
    // ---- reduce-scatter
    for (uint32_t g = g0; g < groups; g += gstep) {
        const uint32_t e = g * L128_ELEMS + ln.elem;
        const bool active = e < Lq;
        u32x4 red = {0u, 0u, 0u, 0u};
        if (active) {
            u32x4 V[NMAX];
#pragma unroll
            for (int s = 0; s < NMAX; ++s)
                if ((uint32_t)s < N)
                    V[s] = ld_elems(inp[s], q * L + e, ln.half);
            Acc8 acc;
#pragma unroll
            for (int s = 0; s < NMAX; ++s)
                if ((uint32_t)s < N) {
                    if (s == 0) acc.init(V[s]); else acc.add(V[s]);
                }
            if constexpr (F32) {
                // debug path: the owner writes its slice's accumulators to every copy
                for (uint32_t r = 0; r < N; ++r)
                    store_lane<true>(a, r, q * L + e, ln.half, acc);
            } else {
                red = acc.bf16();
            }
        }
        if constexpr (!F32)
            l128_publish(stg[q], g * L128_BYTES, lane, ln, red, c.flag);
    }
    if constexpr (F32) {
        finish(a, c);
        return;
    }
    // ---- all-gather
    uint32_t lim[NMAX];
#pragma unroll
    for (int s = 0; s < NMAX; ++s)
        lim[s] = (uint32_t)s < N ? slice_len((uint32_t)s) : 0u;
    char *outq = (char *)a.out + (size_t)q * a.n * 2u;
    const __amdgpu_buffer_rsrc_t oq = rsrc(outq, a.n * 2u);
    for (uint32_t g = g0; g < groups; g += gstep) {
        const uint32_t e = g * L128_ELEMS + ln.elem;
        u32x4 V[NMAX];
        if (!l128_receive<NMAX>(stg, N, (uint32_t)NMAX, g, lane, ln, lim, c.flag, ctl, q,
                                a.watchdog_ticks, V))
            return;
#pragma unroll
        for (int s = 0; s < NMAX; ++s) {
            if ((uint32_t)s < N && e < lim[s]) {
                if (ln.half) {
                    u32x2 p; p.x = V[s].x; p.y = V[s].y;
                    st8<CP_PLAIN>(p, oq, ((uint32_t)s * L + e) * 2u);
                } else {
                    st16<CP_PLAIN>(V[s], oq, ((uint32_t)s * L + e) * 2u);
                }
            }
        }
    }
    finish(a, c);
}

// ==================================================== two-shot sentinel
// Reduce-scatter: rank q pushes chunk c of its slice-s part into inbox
// RS[s][q]; rank s polls RS[s][*], reduces in rank order, re-arms.
// All-gather: rank q pushes its reduced chunk into AG[r][q] of every peer r
// and writes it to out[q]; every rank polls AG[q][*], copies to out, re-arms.
template <int NMAX, bool F32>
__global__ __launch_bounds__(256) void k_twoshot_sentinel(const Launch a)
{
    Ctx0 c;
    c.t0 = clock100();
    c.rank = blockIdx.x % a.n_ranks;
    c.part = blockIdx.x / a.n_ranks;
    const uint32_t N = a.n_ranks;
    const uint32_t q = c.rank;
    const uint32_t L = a.slice;
    const uint32_t G = L >> 3;                      // chunks per slice
    const uint32_t step = a.parts * blockDim.x;
    const uint32_t rounds = (G + step - 1u) / step;
    const uint32_t ibytes = L * 2u;
    uint32_t seq = load_seq(a);
    c.flag = seq + a.epoch;
    c.par = a.epoch & 1u;
    const Ctl ctl{a.ctl};
    const __amdgpu_buffer_rsrc_t inq = in_rsrc(a, q);
    auto rs = [&](uint32_t recv, uint32_t send) {
        return rsrc(a.srs + (size_t)((recv * N + send) * 2u + c.par) * a.s2_stride, ibytes);
    };
    auto ag = [&](uint32_t recv, uint32_t send) {
        return rsrc(a.sag + (size_t)((recv * N + send) * 2u + c.par) * a.s2_stride, ibytes);
    };
    auto slice_len = [&](uint32_t s) -> uint32_t {
        uint32_t lo = s * L;
        return lo >= a.n ? 0u : (a.n - lo < L ? a.n - lo : L);
    };
    const uint32_t Lq = slice_len(q);
    char *outq = (char *)a.out + (size_t)q * a.n * (F32 ? 4u : 2u);
    const __amdgpu_buffer_rsrc_t oq = rsrc(outq, a.n * (F32 ? 4u : 2u));

    for (uint32_t it = 0; it < rounds; ++it) {
        const uint32_t ch = c.part * blockDim.x + threadIdx.x + it * step;
        const uint32_t e = ch * 8u;                 // element offset inside a slice
        // ---- push my parts of every slice
        u32x4 own = {0u, 0u, 0u, 0u};
        u32x4 X[NMAX];
#pragma unroll
        for (int s = 0; s < NMAX; ++s)
            if ((uint32_t)s < N && e < slice_len((uint32_t)s))
                X[s] = ld16<CP_PLAIN>(inq, ((uint32_t)s * L + e) * 2u);
        if (it == 0)
            start_delay(a, c);
#pragma unroll
        for (int s = 0; s < NMAX; ++s) {
            if ((uint32_t)s < N && e < slice_len((uint32_t)s)) {
                if ((uint32_t)s == q) own = X[s];
                else st16<CP_DEV>(X[s], rs((uint32_t)s, q), e * 2u);
            }
        }
        // ---- receive my slice from everyone, reduce, re-arm
        const bool act = e < Lq;
        u32x4 V[NMAX];
        uint32_t pend = 0;
#pragma unroll
        for (int s = 0; s < NMAX; ++s)
            if ((uint32_t)s < N && (uint32_t)s != q && act) {
                V[s] = ld16<CP_DEV>(rs(q, (uint32_t)s), e * 2u);
                pend |= 1u << s;
            }
        Watch w;
        w.begin(a.watchdog_ticks);
        while (true) {
#pragma unroll
            for (int s = 0; s < NMAX; ++s)
                if ((pend >> s) & 1u)
                    if (sent_ready(V[s]))
                        pend &= ~(1u << s);
            if (!wave_any(pend != 0u))
                break;
            if (w.expired(ctl, q, pend ? first_bit(pend) : 0u, c.flag))
                return;
            compiler_fence();
#pragma unroll
            for (int s = 0; s < NMAX; ++s)
                if ((pend >> s) & 1u)
                    V[s] = ld16<CP_DEV>(rs(q, (uint32_t)s), e * 2u);
        }
        if (act) {
            Acc8 acc;
#pragma unroll
            for (int s = 0; s < NMAX; ++s)
                if ((uint32_t)s < N) {
                    u32x4 v = ((uint32_t)s == q) ? own : V[s];
                    if (s == 0) acc.init(v); else acc.add(v);
                }
#pragma unroll
            for (int s = 0; s < NMAX; ++s)
                if ((uint32_t)s < N && (uint32_t)s != q)
                    st16<CP_DEV>(sentinel4(), rs(q, (uint32_t)s), e * 2u);
            if constexpr (F32) {
                // debug path: the owner writes its slice's accumulators to every copy
                for (uint32_t r = 0; r < N; ++r)
                    store_out8<true>(a, r, q * L + e, acc);
            } else {
                const u32x4 red = acc.bf16();
#pragma unroll
                for (int r = 0; r < NMAX; ++r)
                    if ((uint32_t)r < N && (uint32_t)r != q)
                        st16<CP_DEV>(red, ag((uint32_t)r, q), e * 2u);
                store_out8<false>(a, q, q * L + e, acc);
            }
        }
        if constexpr (F32)
            continue;
        // ---- all-gather: receive every other slice's reduced chunk
        pend = 0;
#pragma unroll
        for (int s = 0; s < NMAX; ++s)
            if ((uint32_t)s < N && (uint32_t)s != q && e < slice_len((uint32_t)s)) {
                V[s] = ld16<CP_DEV>(ag(q, (uint32_t)s), e * 2u);
                pend |= 1u << s;
            }
        w.begin(a.watchdog_ticks);
        while (true) {
#pragma unroll
            for (int s = 0; s < NMAX; ++s)
                if ((pend >> s) & 1u)
                    if (sent_ready(V[s]))
                        pend &= ~(1u << s);
            if (!wave_any(pend != 0u))
                break;
            if (w.expired(ctl, q, pend ? first_bit(pend) : 0u, c.flag))
                return;
            compiler_fence();
#pragma unroll
            for (int s = 0; s < NMAX; ++s)
                if ((pend >> s) & 1u)
                    V[s] = ld16<CP_DEV>(ag(q, (uint32_t)s), e * 2u);
        }
#pragma unroll
        for (int s = 0; s < NMAX; ++s)
            if ((uint32_t)s < N && (uint32_t)s != q && e < slice_len((uint32_t)s)) {
                st16<CP_PLAIN>(V[s], oq, ((uint32_t)s * L + e) * 2u);
                st16<CP_DEV>(sentinel4(), ag(q, (uint32_t)s), e * 2u);
            }
    }
    finish(a, c);
}

// ============================================================ maintenance
// Advances the flag sequence after a step of `calls` calls.  When the
// sequence nears the top of its 32-bit range, every flag word is cleared and
// the sequence restarts, so a flag value left in memory long ago can never
// match a future call.
__global__ __launch_bounds__(256) void k_step_end(uint32_t *ctl, uint32_t calls, char *ll,
                                                  size_t ll_bytes, char *l128, size_t l128_bytes)
{
    __shared__ uint32_t wrap;
    if (threadIdx.x == 0) {
        uint32_t s = __hip_atomic_load(ctl + CTL_SEQ, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        uint32_t next = s + calls;
        wrap = (next > 0xFFFE0000u || next < s) ? 1u : 0u;
    }
    __syncthreads();
    if (wrap) {
        uint32_t *w = (uint32_t *)ll;
        for (size_t i = threadIdx.x; i < ll_bytes / 4; i += blockDim.x) w[i] = 0u;
        w = (uint32_t *)l128;
        for (size_t i = threadIdx.x; i < l128_bytes / 4; i += blockDim.x) w[i] = 0u;
        for (uint32_t i = threadIdx.x; i < (uint32_t)MAX_RANKS; i += blockDim.x)
            __hip_atomic_store(ctl + CTL_ARRIVE + 32u * i, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __threadfence();
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t s = __hip_atomic_load(ctl + CTL_SEQ, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(ctl + CTL_SEQ, wrap ? 0u : s + calls, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    }
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

// ------------------------------------------------------------ dispatch
template <int NMAX, bool F32>
static const void *pick(int kind)
{
    switch (kind) {
    case K_ONESHOT_LL: return (const void *)k_oneshot_ll<NMAX, F32>;
    case K_ONESHOT_SENTINEL: return (const void *)k_oneshot_sentinel<NMAX, F32>;
    case K_ONESHOT_DIRECT: return (const void *)k_oneshot_direct<NMAX, F32>;
    case K_ONESHOT_LL128: return (const void *)k_oneshot_ll128<NMAX, F32>;
    case K_TWOSHOT_LL128: return (const void *)k_twoshot_ll128<NMAX, F32>;
    case K_TWOSHOT_SENTINEL: return (const void *)k_twoshot_sentinel<NMAX, F32>;
    default: return nullptr;
    }
}

const void *kernel_for(int kind, int n_ranks, bool f32)
{
    if (n_ranks <= 8)
        return f32 ? pick<8, true>(kind) : pick<8, false>(kind);
    return f32 ? pick<16, true>(kind) : pick<16, false>(kind);
}

hipError_t launch_ar(int kind, bool f32, const Launch &a, uint32_t grid, uint32_t threads,
                     hipStream_t stream)
{
    const void *fn = kernel_for(kind, (int)a.n_ranks, f32);
    if (fn == nullptr)
        return hipErrorInvalidValue;
    void *args[] = {(void *)&a};
    return hipLaunchKernel(fn, dim3(grid), dim3(threads), args, 0, stream);
}

hipError_t launch_step_end(uint32_t *ctl, uint32_t calls, char *ll, size_t ll_bytes, char *l128,
                           size_t l128_bytes, hipStream_t stream)
{
    hipLaunchKernelGGL(k_step_end, dim3(1), dim3(256), 0, stream, ctl, calls, ll, ll_bytes, l128,
                       l128_bytes);
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
