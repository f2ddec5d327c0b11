// ar_host.hip -- host side of the C ABI declared in include/ar.h.
//
// Owns the single process-wide context: staging for every protocol (per
// rank x 2 parities), the control block (flag-sequence base, status record,
// arrival flags), launch geometry, the epoch sequence check and the
// algorithm/protocol choice (the pages' table of variants, "微秒必争…",
// section "统一原语与API设计", re-measured for this chip: see oneshot_limit).
#include <hip/hip_runtime.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>
#include <strings.h>

#include <algorithm>
#include <cmath>
#include <vector>

#include "../../include/ar.h"
#include "ar_kernels.h"
#include "ar_proto.h"

namespace {

using ar::Launch;

constexpr size_t MAX_ELEMS_LIMIT = size_t(1) << 28;
constexpr uint32_t DEFAULT_WATCHDOG_US = 200000;
// Automatic selection by per-rank message size S = 2n bytes, from a sweep
// of every algorithm/protocol pair on MI355X (8 ranks, 4 KiB - 4 MiB, graphs
// of 40 calls).  The pages' table (one-shot below 64 KB, two-shot above) was
// drawn for NVLink; here the in-place one-shot stays ahead much longer:
//   one-shot DIRECT below 1 MiB (4 KiB: 2.51 us vs 2.59 one-shot LL;
//   16 KiB: 2.60 vs 2.72; 256 KiB: 3.63 vs 5.41 two-shot DIRECT),
//   two-shot DIRECT from 1 MiB (1 MiB: 5.99 vs 7.18; 4 MiB: 12.99 vs 24.52).
// With a protocol fixed and the algorithm left to AUTO, the one-shot limit
// is that protocol's own crossover.
// The fused AllReduce + norm keeps its LL form up to 16 KiB (its in-place
// form was not re-measured against it after the prologue changes).
constexpr size_t AUTO_NORM_LL_MAX_BYTES = 16 * 1024;
constexpr uint64_t ONESHOT_DIRECT_MAX_PARTS = 128;
// Largest per-rank message (bytes) for which the in-place one-shot gives each
// lane 4 elements instead of 8 (latency-bound sizes, where the fold's
// instruction count per lane shows).
constexpr size_t ONESHOT_UNIT4_MAX_BYTES = 64 * 1024;
// rate of the constant clock the kernels' timers count (100 MHz)
constexpr int WALL_CLOCK_KHZ = 100000;
// Fixed-size staging (the double buffering of "微秒必争…", section
// "四大核心机制", item 3; NCCL's bounded NCCL_BUFFSIZE on the "vLLM 分布式推理
// 核心" page, section 四): each staged protocol gets a window per rank (LL,
// LL128) or per (receiver, sender) pair (sentinel inboxes) and buffer, at
// most these sizes, whatever max_elems is; larger messages are walked in
// rounds through the two buffers.  One round of one part takes 1 KiB of a
// window (LL: 64 chunks of 4 elements as 16-byte units; sentinel: 64 chunks
// of 8 elements; LL128: one 1-KiB line group per wave of the batch).
constexpr size_t STAGE_WINDOW_MAX = 1024 * 1024;       // LL, LL128: per rank and buffer
constexpr size_t STAGE_INBOX_MAX = 256 * 1024;         // sentinel: per pair and buffer
constexpr size_t STAGE_ROUND_BYTES = 1024;             // one part's round (per line group for LL128)
constexpr size_t STAGE_WINDOW_MIN = 4096;              // a whole LL128 batch of 4 groups
// A window holds whole rounds of a multiple of 8 parts (the part count is
// rounded up to one, so that part p runs on XCD p % 8): windows are sized in
// multiples of 8 part-rounds (LL128: of batches of 4 groups).
constexpr size_t STAGE_QUANTUM = 8 * STAGE_ROUND_BYTES;
constexpr size_t STAGE_QUANTUM_L128 = 8 * 4 * STAGE_ROUND_BYTES;
size_t oneshot_limit(int proto)
{
    switch (proto) {
    case AR_PROTO_SENTINEL: return 64 * 1024;          // two-shot ahead from 128 KiB
    case AR_PROTO_LL128: return 128 * 1024;            // two-shot ahead from 256 KiB
    default: return 1024 * 1024 - 1;                   // DIRECT, barrier, AUTO
    }
}

struct Context {
    bool live = false;
    int device = -1;
    int n_ranks = 0;
    size_t max_elems = 0;
    int cu_count = 0;
    int wall_khz = 0;   // constant-clock rate (hipDeviceAttributeWallClockRate)
    // staging
    char *ll = nullptr;   size_t ll_stride = 0;
    char *l128 = nullptr; size_t l128_stride = 0;
    char *s1 = nullptr;   size_t s1_stride = 0;
    char *srs = nullptr;  char *sag = nullptr; size_t s2_stride = 0;
    uint32_t *ctl = nullptr;
    uint32_t *done = nullptr;           // two-shot DIRECT completion flags
    uint32_t *stats = nullptr;          // fused norm: per-block sums of squares {sum, flag}
    char *acc = nullptr;  size_t acc_stride = 0;   // atomic lines, per parity
    size_t stats_stride = 0;            // entries per rank
    size_t window = 0;                  // staging window in use (0: the whole allocation)
    // options
    int algo = AR_ALGO_AUTO;
    int proto = AR_PROTO_AUTO;
    int wgs_per_rank = 0;
    int scope = AR_SCOPE_AUTO;
    bool placement_ok = false;   // round-robin XCD dispatch verified at init
    int threads = 0;                    // 0 = chosen per call
    uint32_t watchdog_us = DEFAULT_WATCHDOG_US;
    const uint32_t *delays = nullptr; size_t delay_rows = 0;
    uint64_t *ts = nullptr; size_t ts_slots = 0, ts_stride = 0; bool ts_phases = false;
    // sequence
    uint32_t last_epoch = 0;
    uint64_t step_rounds = 0;           // rounds of the current step's calls so far
    int capacity[ar::K_COUNT][2][5] = {};   // resident workgroups [kind][f32][64..1024 threads]
    int cap_l128[2][2][3] = {};             // LL128 at 256 threads [two-shot][f32][1, 2, 4 groups]
    bool cap_ready = false;
};

Context g;
int g_last_hip = 0;

int hip_fail(hipError_t e)
{
    g_last_hip = (int)e;
    return AR_ERR_HIP;
}

// Start-up defaults from the environment (read by ar_init, as NCCL reads
// NCCL_ALGO / NCCL_PROTO): AR_ALGO = auto | oneshot | twoshot, AR_PROTO =
// auto | ll | ll128 | sentinel | direct | barrier | atomic, AR_WATCHDOG_MS =
// a positive integer.  A value that does not parse, or an impossible
// algorithm/protocol pair, makes ar_init fail with AR_ERR_INVALID.
int env_choice(const char *name, const char *const *names, int count, int *out)
{
    const char *e = getenv(name);
    if (e == nullptr || *e == 0)
        return AR_OK;
    for (int i = 0; i < count; ++i)
        if (strcasecmp(e, names[i]) == 0) {
            *out = i;
            return AR_OK;
        }
    return AR_ERR_INVALID;
}

int apply_env(int *algo, int *proto, uint32_t *watchdog_us)
{
    static const char *const algos[] = {"auto", "oneshot", "twoshot"};
    static const char *const protos[] = {"auto", "ll", "ll128", "sentinel", "direct", "barrier",
                                         "atomic"};
    int rc = env_choice("AR_ALGO", algos, 3, algo);
    if (rc == AR_OK)
        rc = env_choice("AR_PROTO", protos, 7, proto);
    if (rc != AR_OK)
        return rc;
    if ((*algo == AR_ALGO_TWOSHOT && *proto == AR_PROTO_LL) ||
        (*algo == AR_ALGO_ONESHOT && *proto == AR_PROTO_ATOMIC))
        return AR_ERR_INVALID;
    const char *w = getenv("AR_WATCHDOG_MS");
    if (w != nullptr && *w != 0) {
        char *end = nullptr;
        const long ms = strtol(w, &end, 10);
        if (end == w || *end != 0 || ms <= 0 || ms > 4000000)
            return AR_ERR_INVALID;
        *watchdog_us = (uint32_t)ms * 1000u;
    }
    return AR_OK;
}

bool debug_enabled()
{
    static int v = -1;
    if (v < 0) {
        const char *e = getenv("AR_DEBUG");
        v = (e && *e && strcmp(e, "0") != 0) ? 1 : 0;
    }
    return v == 1;
}

size_t round_up(size_t x, size_t m) { return (x + m - 1) / m * m; }

size_t slice_len(size_t n, int n_ranks) { return round_up((n + n_ranks - 1) / n_ranks, 8); }

void free_all()
{
    char **bufs[] = {&g.ll, &g.l128, &g.s1, &g.srs, &g.sag, &g.acc};
    for (char **b : bufs) {
        if (*b) (void)hipFree(*b);
        *b = nullptr;
    }
    g.ctl = nullptr;                    // the device's static control block
    if (g.done) (void)hipFree(g.done);
    g.done = nullptr;
    if (g.stats) (void)hipFree(g.stats);
    g.stats = nullptr;
}

constexpr size_t REGION_LIMIT = (size_t(1) << 32) - 1;   // one buffer descriptor

int alloc(char **p, size_t bytes)
{
    hipError_t e = hipMalloc((void **)p, bytes);
    if (e == hipErrorOutOfMemory || e == hipErrorMemoryAllocation) {
        *p = nullptr;
        g_last_hip = (int)e;
        return AR_ERR_OOM;
    }
    if (e != hipSuccess) {
        *p = nullptr;
        return hip_fail(e);
    }
    return AR_OK;
}

size_t ll_bytes() { return g.ll_stride * 2 * g.n_ranks; }
size_t l128_bytes() { return g.l128_stride * 2 * g.n_ranks; }
size_t s1_bytes() { return g.s1_stride * 2 * g.n_ranks * g.n_ranks; }
size_t s2_bytes() { return g.s2_stride * 2 * g.n_ranks * g.n_ranks; }
size_t done_words() { return (size_t)ar::MAX_RANKS * ar::DONE_STRIDE; }
size_t stats_bytes() { return g.stats_stride * 8 * g.n_ranks; }
size_t acc_bytes() { return g.acc_stride * 2; }

// Zero flags, arm sentinels, clear the control block -- kernels only.
hipError_t rearm(hipStream_t s)
{
    hipError_t e;
    if ((e = ar::launch_fill((uint32_t *)g.ll, ll_bytes() / 4, 0u, s)) != hipSuccess) return e;
    if ((e = ar::launch_fill((uint32_t *)g.l128, l128_bytes() / 4, 0u, s)) != hipSuccess) return e;
    if (g.s1 && (e = ar::launch_fill((uint32_t *)g.s1, s1_bytes() / 4, ar::SENT_WORD, s)) != hipSuccess) return e;
    if ((e = ar::launch_fill((uint32_t *)g.srs, s2_bytes() / 4, ar::SENT_WORD, s)) != hipSuccess) return e;
    if ((e = ar::launch_fill((uint32_t *)g.sag, s2_bytes() / 4, ar::SENT_WORD, s)) != hipSuccess) return e;
    if ((e = ar::launch_fill(g.done, done_words(), 0u, s)) != hipSuccess) return e;
    if ((e = ar::launch_fill(g.stats, stats_bytes() / 4, 0u, s)) != hipSuccess) return e;
    if ((e = ar::launch_fill((uint32_t *)g.acc, acc_bytes() / 4, 0u, s)) != hipSuccess) return e;
    return ar::launch_fill(g.ctl, ar::CTL_WORDS, 0u, s);
}

int thread_index(int threads)
{
    return threads <= 64 ? 0 : threads <= 128 ? 1 : threads <= 256 ? 2 : threads <= 512 ? 3 : 4;
}

int compute_capacity()
{
    // The capacity of a kind is the minimum over the kernels a call of it may
    // launch: both coherence scopes (bf16) and the test twins (bf16),
    // so a grid sized by it is resident at once whichever runs.
    const int tcounts[5] = {64, 128, 256, 512, 1024};
    auto occupancy = [](const void *fn, int threads, int *per_cu) -> hipError_t {
        *per_cu = 0;
        return hipOccupancyMaxActiveBlocksPerMultiprocessor(per_cu, fn, threads, 0);
    };
    for (int k = 0; k < ar::K_COUNT; ++k) {
        for (int f = 0; f < 2; ++f) {
            if (ar::kernel_for(k, g.n_ranks, f == 1, false, 0) == nullptr)
                continue;                       // no such variant (capacity stays 0)
            for (int t = 0; t < 5; ++t) {
                int best = 1 << 30;
                bool usable = true;
                for (int v = 0; v < (f == 0 ? 6 : 1) && usable; ++v) {
                    int per_cu = 0;
                    const void *fn = ar::kernel_for(k, g.n_ranks, f == 1, (v & 1) != 0, 0, v >> 1);
                    hipError_t e = occupancy(fn, tcounts[t], &per_cu);
                    if (e != hipSuccess && t >= 3) {
                        // block sizes above a kernel's launch bound: unusable
                        (void)hipGetLastError();
                        usable = false;
                    } else if (e != hipSuccess) {
                        return hip_fail(e);
                    }
                    best = std::min(best, per_cu);
                }
                g.capacity[k][f][t] = usable ? best * g.cu_count : 0;
            }
        }
    }
    // LL128 per batch size (its LDS tile grows with the groups per batch)
    const int gws[3] = {1, 2, 4};
    for (int two = 0; two < 2; ++two)
        for (int f = 0; f < 2; ++f)
            for (int i = 0; i < 3; ++i) {
                const int kind = two ? ar::K_TWOSHOT_LL128 : ar::K_ONESHOT_LL128;
                int best = 1 << 30;
                for (int v = 0; v < (f ? 1 : 6); ++v) {
                    int per_cu = 0;
                    hipError_t e = occupancy(ar::kernel_for(kind, g.n_ranks, f == 1, (v & 1) != 0,
                                                            gws[i], v >> 1),
                                             256, &per_cu);
                    if (e != hipSuccess)
                        return hip_fail(e);
                    best = std::min(best, per_cu);
                }
                g.cap_l128[two][f][i] = best * g.cu_count;
            }
    g.cap_ready = true;
    return AR_OK;
}

struct Plan {
    int kind;
    int gw = 0;         // LL128: line groups per batch
    uint32_t parts;     // workgroups per rank
    uint32_t threads;
    uint32_t slice;
    bool local;         // XCD-local coherence scope
    bool rank_xcd = false; // grid (1, N, parts): rank r on XCD r mod 8 (cross-XCD exchanges)
    bool unit4 = false; // in-place one-shot: 4-element lane units
    uint32_t rounds = 1; // rounds of the call (each takes its own flag)
};

uint64_t ceil_div(uint64_t a, uint64_t b) { return (a + b - 1) / b; }

// The staging window a kind walks its rounds through (bytes per rank, or per
// inbox pair, and buffer), 0 for kinds without staging.
size_t window_of(int kind)
{
    size_t alloc = 0;
    switch (kind) {
    case ar::K_ONESHOT_LL:
    case ar::K_ONESHOT_LL_NORM: alloc = g.ll_stride; break;
    case ar::K_ONESHOT_LL128:
    case ar::K_TWOSHOT_LL128: alloc = g.l128_stride; break;
    case ar::K_ONESHOT_SENTINEL: alloc = g.s1_stride; break;
    case ar::K_TWOSHOT_SENTINEL: alloc = g.s2_stride; break;
    default: return 0;
    }
    return g.window != 0 && g.window < alloc ? g.window : alloc;
}

// Rounds a call walks: the loop count of its part 0 (every part walks at
// most as many).  Kinds without rounds take one flag.
uint32_t rounds_of(const Plan &p, size_t n)
{
    uint64_t r = 1;
    switch (p.kind) {
    case ar::K_ONESHOT_LL:
    case ar::K_ONESHOT_LL_NORM: r = ceil_div(n / 4, (uint64_t)p.parts * 64); break;
    case ar::K_ONESHOT_SENTINEL: r = ceil_div(n / 8, (uint64_t)p.parts * 64); break;
    case ar::K_TWOSHOT_SENTINEL: r = ceil_div(p.slice / 8, (uint64_t)p.parts * 64); break;
    case ar::K_ONESHOT_LL128:
        r = ceil_div(ceil_div(ceil_div(n, ar::L128_ELEMS), (uint64_t)p.gw), p.parts); break;
    case ar::K_TWOSHOT_LL128:
        r = ceil_div(ceil_div(ceil_div(p.slice, ar::L128_ELEMS), (uint64_t)p.gw), p.parts); break;
    default: break;
    }
    return r == 0 ? 1u : (uint32_t)r;
}

int choose_kind(size_t n, int *kind)
{
    const size_t bytes = 2 * n;
    int algo = g.algo, proto = g.proto;
    if (algo == AR_ALGO_AUTO) {
        if (proto == AR_PROTO_LL)
            algo = AR_ALGO_ONESHOT;
        else if (proto == AR_PROTO_ATOMIC)
            algo = AR_ALGO_TWOSHOT;
        else
            algo = bytes <= oneshot_limit(proto) ? AR_ALGO_ONESHOT : AR_ALGO_TWOSHOT;
    }
    if (proto == AR_PROTO_AUTO)
        proto = AR_PROTO_DIRECT;
    if (algo == AR_ALGO_ONESHOT) {
        switch (proto) {
        case AR_PROTO_LL: *kind = ar::K_ONESHOT_LL; return AR_OK;
        case AR_PROTO_LL128: *kind = ar::K_ONESHOT_LL128; return AR_OK;
        case AR_PROTO_SENTINEL:
            *kind = ar::K_ONESHOT_SENTINEL; return AR_OK;
        case AR_PROTO_DIRECT: *kind = ar::K_ONESHOT_DIRECT; return AR_OK;
        case AR_PROTO_BARRIER: *kind = ar::K_ONESHOT_BARRIER; return AR_OK;
        default: break;                 // the atomic lines are a two-phase algorithm
        }
    } else {
        switch (proto) {
        case AR_PROTO_LL128: *kind = ar::K_TWOSHOT_LL128; return AR_OK;
        case AR_PROTO_SENTINEL: *kind = ar::K_TWOSHOT_SENTINEL; return AR_OK;
        case AR_PROTO_DIRECT: *kind = ar::K_TWOSHOT_DIRECT; return AR_OK;
        case AR_PROTO_BARRIER: *kind = ar::K_TWOSHOT_BARRIER; return AR_OK;
        case AR_PROTO_ATOMIC: *kind = ar::K_TWOSHOT_ATOMIC; return AR_OK;
        }
    }
    return AR_ERR_INVALID;
}

// Launch geometry.  Work unit per kind: a lane chunk of 4 elements (LL; the
// DIRECT one-shot up to 64 KiB per rank), of 8 elements (sentinel; the
// DIRECT one-shot above that), two 8-element chunks (DIRECT two-shot), or a
// wave-wide LL128 line group of 480 elements.  Small
// messages use one-wave workgroups spread over many CUs (each CU then polls
// little); large ones use 4-wave workgroups.  The whole grid must be
// resident at once.
int plan_geometry(size_t n, bool f32, Plan *p)
{
    int rc;
    const uint32_t N = (uint32_t)g.n_ranks;
    p->slice = (uint32_t)slice_len(n, g.n_ranks);
    const bool l128 = p->kind == ar::K_ONESHOT_LL128 || p->kind == ar::K_TWOSHOT_LL128;
    if (l128) {
        // line groups per batch, from sweeps at 8 ranks (ar_kernels.hip; the
        // one-shot from 1 MiB per rank: 4 against 2, 14.75 -> 13.4 us at
        // 1 MiB, 24.4 -> 21.2 at 2 MiB, 43.2 -> 37.6 at 4 MiB)
        const size_t bytes = 2 * n;
        if (p->kind == ar::K_ONESHOT_LL128)
            p->gw = bytes <= 64 * 1024 ? 1 : (bytes <= 512 * 1024 || N > 8) ? 2 : 4;
        else
            p->gw = bytes <= 1024 * 1024 ? 1 : (N <= 8 ? 4 : 2);
    }
    if (p->kind == ar::K_ONESHOT_LL || p->kind == ar::K_ONESHOT_LL_NORM) {
        // one wave per rank (a power of two >= N): each wave receives one peer
        uint32_t w = 1;
        while (w < N) w <<= 1;
        p->threads = 64 * w;
    } else if (p->kind == ar::K_ONESHOT_SENTINEL || p->kind == ar::K_TWOSHOT_SENTINEL)
        p->threads = 512;               // 8 waves share the peers of a tile
    else if (l128)
        p->threads = 256;               // 4 waves share the peers of a tile
    else if (g.threads > 0)
        p->threads = (uint32_t)g.threads;
    else if (l128 || p->kind == ar::K_TWOSHOT_DIRECT || p->kind == ar::K_TWOSHOT_BARRIER ||
             p->kind == ar::K_TWOSHOT_ATOMIC || p->kind == ar::K_ONESHOT_DIRECT_NORM)
        p->threads = 256;
    else
        p->threads = 2 * n <= 256 * 1024 ? 64 : 256;
    uint64_t units, per_wg;
    switch (p->kind) {
    case ar::K_ONESHOT_LL:
    case ar::K_ONESHOT_LL_NORM:
        units = n / 4; per_wg = 64; break;
    case ar::K_ONESHOT_LL128:       // batches of gw line groups (at most 2 above 8 ranks)
        units = (n + ar::L128_ELEMS - 1) / ar::L128_ELEMS; per_wg = (uint64_t)p->gw; break;
    case ar::K_TWOSHOT_LL128:
        units = (p->slice + ar::L128_ELEMS - 1) / ar::L128_ELEMS; per_wg = (uint64_t)p->gw; break;
    case ar::K_ONESHOT_SENTINEL:
        units = n / 8; per_wg = 64; break;
    case ar::K_TWOSHOT_SENTINEL:
        units = p->slice / 8; per_wg = 64; break;
    case ar::K_TWOSHOT_DIRECT:       // the barrier-ful baseline shares its data phase
    case ar::K_TWOSHOT_BARRIER:
        units = p->slice / 8; per_wg = ar::TWOSHOT_DIRECT_CHUNKS * p->threads; break;
    case ar::K_ONESHOT_DIRECT_NORM: // one 256-element norm block per wave
        units = n / ar::NORM_BLOCK_ELEMS; per_wg = p->threads / 64; break;
    case ar::K_TWOSHOT_ATOMIC:      // lines of 31 elements, two per wave
        units = (n + ar::ATOM_LINE_ELEMS - 1) / ar::ATOM_LINE_ELEMS; per_wg = p->threads / 32; break;
    case ar::K_ONESHOT_DIRECT:      // the barrier-ful baseline shares its data phase
    case ar::K_ONESHOT_BARRIER:
        p->unit4 = 2 * n <= ONESHOT_UNIT4_MAX_BYTES;
        units = p->unit4 ? n / 4 : n / 8; per_wg = p->threads; break;
    default:
        units = n / 8; per_wg = p->threads; break;
    }
    if (!g.cap_ready) {
        rc = compute_capacity();
        if (rc != AR_OK)
            return rc;
    }
    uint32_t cap = (uint32_t)g.capacity[p->kind][f32 ? 1 : 0][thread_index((int)p->threads)] / N;
    if (l128)
        cap = (uint32_t)g.cap_l128[p->kind == ar::K_TWOSHOT_LL128][f32 ? 1 : 0]
                                  [p->gw == 1 ? 0 : p->gw == 2 ? 1 : 2] / N;
    if (cap > ar::DONE_STRIDE)
        cap = ar::DONE_STRIDE;
    if (p->kind == ar::K_ONESHOT_BARRIER || p->kind == ar::K_TWOSHOT_BARRIER ||
        p->kind == ar::K_ONESHOT_LL_NORM || p->kind == ar::K_ONESHOT_DIRECT_NORM) {
        // a grid barrier (or the norm's row-wide wait) needs every workgroup
        // resident at once: stay within half the occupancy-derived capacity
        // (the watchdog bounds the rest)
        cap /= 2;
        if (cap > ar::DONE_STRIDE)
            cap = ar::DONE_STRIDE;
    }
    // one round of every part must fit the staging window
    const size_t win = window_of(p->kind);
    if (win != 0) {
        const size_t round_bytes = STAGE_ROUND_BYTES * (l128 ? (size_t)p->gw : 1);
        const size_t win_parts = win / round_bytes;
        if (win_parts < cap)
            cap = (uint32_t)win_parts;
    }
    if (cap == 0)
        return AR_ERR_INVALID;
    uint64_t want = g.wgs_per_rank > 0 ? (uint64_t)g.wgs_per_rank : (units + per_wg - 1) / per_wg;
    if (want == 0) want = 1;
    if (g.wgs_per_rank == 0) {
        // a multiple of the XCD count puts part p of every rank on XCD p % 8
        // (round-robin dispatch), so each part's exchange stays in one L2;
        // surplus workgroups find no work and only take part in the flags
        const uint64_t X = ar::XCDS;
        const uint64_t up = (want + X - 1) / X * X;
        if (up <= cap)
            want = up;
        else if (cap >= X)
            want = cap / X * X;
    }
    if (want > cap) want = cap;
    // the in-place one-shot loops rather than spreading wider: beyond 128
    // workgroups of 256 threads per rank the N-fold reads of a chunk crowd
    // the L2 (1 MiB per rank: 6.4 us at 128 vs 7.2 at 256)
    if (p->kind == ar::K_ONESHOT_DIRECT && g.wgs_per_rank == 0 && p->threads == 256 &&
        want > ONESHOT_DIRECT_MAX_PARTS)
        want = ONESHOT_DIRECT_MAX_PARTS;
    p->parts = (uint32_t)want;
    p->local = !f32 && g.scope == AR_SCOPE_AUTO && g.placement_ok && p->parts % ar::XCDS == 0;
    p->rank_xcd = g.scope == AR_SCOPE_CROSS_XCD;
    p->rounds = rounds_of(*p, n);
    return AR_OK;
}

int make_plan(size_t n, bool f32, Plan *p)
{
    int rc = choose_kind(n, &p->kind);
    if (rc != AR_OK)
        return rc;
    return plan_geometry(n, f32, p);
}

int check_call(const void *const *rank_bufs, const void *out, size_t out_elem_bytes, size_t n,
               uint32_t epoch)
{
    if (!g.live)
        return AR_ERR_NOT_INIT;
    if (rank_bufs == nullptr || out == nullptr)
        return AR_ERR_INVALID;
    if (n == 0 || n > g.max_elems || (n % 8) != 0)
        return AR_ERR_INVALID;
    if (epoch == 0 || epoch > 0xFFFFu || epoch != g.last_epoch + 1)
        return AR_ERR_INVALID;
    const uintptr_t o = (uintptr_t)out;
    if (o % 16)
        return AR_ERR_INVALID;
    const uintptr_t o_end = o + out_elem_bytes * n * (size_t)g.n_ranks;
    for (int r = 0; r < g.n_ranks; ++r) {
        const uintptr_t b = (uintptr_t)rank_bufs[r];
        if (b == 0 || b % 16)
            return AR_ERR_INVALID;
        const uintptr_t b_end = b + 2 * n;
        if (b < o_end && o < b_end)
            return AR_ERR_INVALID;      // output overlaps an input
    }
    return AR_OK;
}

// Checks that a launch's workgroups are dealt to the 8 XCDs round-robin:
// the workgroup with linear index b on XCD (b + o) % 8 for one offset o per
// launch, for both workgroup sizes in use and for a flat grid as well as
// the AllReduce grid shape (8, N, blocks).  The XCD-local scope is only
// enabled if so.
hipError_t verify_placement(bool *ok)
{
    *ok = false;
    const uint32_t grid = 4096;
    uint32_t *d = nullptr;
    hipError_t e = hipMalloc((void **)&d, grid * 4);
    if (e != hipSuccess)
        return e;
    std::vector<uint32_t> h(grid);
    bool good = true;
    const uint32_t N = (uint32_t)g.n_ranks;
    const uint32_t shapes[3][3] = {{grid, 1, 1}, {ar::XCDS, N, grid / (ar::XCDS * N)},
                                   {1, N, grid / N}};
    for (const auto &sh : shapes) {
        const uint32_t total = sh[0] * sh[1] * sh[2];
        for (uint32_t threads : {64u, 256u}) {
            if ((e = ar::launch_fill(d, grid, 0xFFFFFFFFu, 0)) != hipSuccess ||
                (e = ar::launch_xcc_map(d, sh[0], sh[1], sh[2], threads, 0)) != hipSuccess ||
                (e = hipMemcpy(h.data(), d, grid * 4, hipMemcpyDeviceToHost)) != hipSuccess)
                break;
            uint32_t bad = 0, first = total;
            const uint32_t o = h[0] % ar::XCDS;
            for (uint32_t b = 0; b < total; ++b)
                if (h[b] != (b + o) % ar::XCDS) {
                    ++bad;
                    if (first == total) first = b;
                }
            if (bad && debug_enabled())
                fprintf(stderr, "[ar] placement check (grid %ux%ux%u, %u threads): %u of %u "
                        "workgroups off the round-robin order (offset %u), first b=%u on XCD %u\n",
                        sh[0], sh[1], sh[2], threads, bad, total, o, first, h[first]);
            good = good && bad == 0;
        }
        if (e != hipSuccess)
            break;
    }
    hipError_t ef = hipFree(d);
    if (e == hipSuccess)
        e = ef;
    *ok = e == hipSuccess && good;
    return e;
}

void fill_launch(const void *const *rank_bufs, void *out, size_t n, uint32_t epoch, const Plan &p,
                 Launch *ap)
{
    Launch &a = *ap;
    memset(&a, 0, sizeof a);
    for (int r = 0; r < g.n_ranks; ++r)
        a.in[r] = rank_bufs[r];
    a.out = out;
    a.ll = g.ll; a.l128 = g.l128; a.s1 = g.s1; a.srs = g.srs; a.sag = g.sag;
    a.ctl = g.ctl;
    a.done = g.done;
    a.acc = g.acc; a.acc_stride = (uint32_t)g.acc_stride;
    a.ts = g.ts; a.ts_slots = (uint32_t)g.ts_slots; a.ts_stride = (uint32_t)g.ts_stride;
    a.ts_phases = g.ts_phases ? 1u : 0u;
    a.delays = g.delays; a.delay_rows = (uint32_t)g.delay_rows;
    a.ll_stride = (uint32_t)g.ll_stride; a.l128_stride = (uint32_t)g.l128_stride;
    a.s1_stride = (uint32_t)g.s1_stride; a.s2_stride = (uint32_t)g.s2_stride;
    a.n = (uint32_t)n;
    a.n_ranks = (uint32_t)g.n_ranks;
    a.epoch = epoch;
    a.rbase = (uint32_t)g.step_rounds;
    a.parts = p.parts;
    a.slice = p.slice;
    // workgroup layout: grid (8, N, parts / 8) when parts % 8 == 0 (blocks
    // of 8 parts x N ranks, so part p runs on XCD p % 8), else -- and always
    // for the cross-XCD scope -- (1, N, parts): workgroup (r, p) has linear
    // index r + N p, so with 8 ranks rank r runs on XCD r (with 4, on XCDs
    // r and r + 4; with 16, ranks r and r + 8 share XCD r mod 8)
    a.xshift = !p.rank_xcd && p.parts % ar::XCDS == 0 ? 3u : 0u;
    a.unit4 = p.unit4 ? 1u : 0u;
    uint64_t ticks = (uint64_t)g.watchdog_us * 100u;   // 100 MHz clock
    a.watchdog_ticks = (uint32_t)std::min<uint64_t>(ticks, 0xFFFFFFFFu);
}

int do_allreduce(const void *const *rank_bufs, void *out, size_t n, uint32_t epoch,
                 hipStream_t stream, bool f32)
{
    int rc = check_call(rank_bufs, out, f32 ? 4 : 2, n, epoch);
    if (rc != AR_OK)
        return rc;
    Plan p;
    rc = make_plan(n, f32, &p);
    if (rc != AR_OK)
        return rc;
    if (g.step_rounds + p.rounds > ar::STEP_ROUNDS_MAX)
        return AR_ERR_INVALID;          // close the step with ar_step_end first
    Launch a;
    fill_launch(rank_bufs, out, n, epoch, p, &a);
    const uint32_t grid = p.parts * (uint32_t)g.n_ranks;
    if (debug_enabled())
        fprintf(stderr, "[ar] n=%zu epoch=%u kind=%d grid=%u threads=%u slice=%u rounds=%u f32=%d "
                "local=%d\n", n, epoch, p.kind, grid, p.threads, p.slice, p.rounds, (int)f32,
                (int)p.local);
    hipError_t e = ar::launch_ar(p.kind, f32, p.local, p.gw, a, p.threads, stream);
    if (e != hipSuccess)
        return hip_fail(e);
    g.last_epoch = epoch;
    g.step_rounds += p.rounds;
    return AR_OK;
}


bool overlap(const void *a, size_t an, const void *b, size_t bn)
{
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return x < y + bn && y < x + an;
}

// Checks of the residual add + RMS norm operands shared by the fused and
// the stand-alone entry points: rows x hidden per rank, hidden a multiple of
// 256 up to 65536, 16-byte aligned operands, outputs h and y [N][n] disjoint
// from each other and from every operand read (src [N] arrays of n elements,
// residuals, gamma).
int check_norm(const void *const *src, size_t src_count, const void *const *residual,
               const void *gamma, float eps, const void *out_h, const void *out_y, size_t rows,
               size_t hidden, size_t *n_out)
{
    if (residual == nullptr || gamma == nullptr || out_h == nullptr || out_y == nullptr ||
        src == nullptr)
        return AR_ERR_INVALID;
    if (hidden < ar::NORM_BLOCK_ELEMS || hidden % ar::NORM_BLOCK_ELEMS != 0 ||
        hidden > ar::NORM_HIDDEN_LIMIT || rows == 0 || rows > g.max_elems / hidden)
        return AR_ERR_INVALID;
    if (!std::isfinite(eps) || eps < 0.0f)
        return AR_ERR_INVALID;
    const size_t n = rows * hidden;
    const size_t out_bytes = 2 * n * (size_t)g.n_ranks;
    const void *ptrs[] = {gamma, out_h, out_y};
    for (const void *q : ptrs)
        if ((uintptr_t)q % 16)
            return AR_ERR_INVALID;
    if (overlap(out_h, out_bytes, out_y, out_bytes) || overlap(out_h, out_bytes, gamma, 2 * hidden) ||
        overlap(out_y, out_bytes, gamma, 2 * hidden))
        return AR_ERR_INVALID;
    for (int r = 0; r < g.n_ranks; ++r) {
        const void *q = residual[r];
        if (q == nullptr || (uintptr_t)q % 16 || overlap(out_h, out_bytes, q, 2 * n) ||
            overlap(out_y, out_bytes, q, 2 * n))
            return AR_ERR_INVALID;
    }
    for (size_t r = 0; r < src_count; ++r) {
        const void *q = src[r];
        const size_t len = src_count == 1 ? out_bytes : 2 * n;
        if (q == nullptr || (uintptr_t)q % 16 || overlap(out_h, out_bytes, q, len) ||
            overlap(out_y, out_bytes, q, len))
            return AR_ERR_INVALID;
    }
    *n_out = n;
    return AR_OK;
}

int do_allreduce_norm(const void *const *rank_bufs, const void *const *residual, const void *gamma,
                      float eps, void *out_h, void *out_y, size_t rows, size_t hidden,
                      uint32_t epoch, hipStream_t stream)
{
    if (!g.live)
        return AR_ERR_NOT_INIT;
    size_t n = 0;
    int rc = check_norm(rank_bufs, (size_t)g.n_ranks, residual, gamma, eps, out_h, out_y, rows,
                        hidden, &n);
    if (rc != AR_OK)
        return rc;
    rc = check_call(rank_bufs, out_h, 2, n, epoch);
    if (rc != AR_OK)
        return rc;
    // the fused epilogue rides on the one-shot LL or the in-place one-shot:
    // LL for messages up to 16 KiB, DIRECT above (or as the protocol option
    // fixes it); no other protocol has a fused form.  The
    // in-place form goes row-wise (a workgroup per rank and row) for 8 or
    // more rows of up to 8192 elements when they fit the device at once.
    Plan p;
    if (g.proto == AR_PROTO_LL || (g.proto == AR_PROTO_AUTO && 2 * n <= AUTO_NORM_LL_MAX_BYTES))
        p.kind = ar::K_ONESHOT_LL_NORM;
    else if (g.proto == AR_PROTO_AUTO || g.proto == AR_PROTO_DIRECT)
        p.kind = ar::K_ONESHOT_DIRECT_NORM;
    else
        return AR_ERR_INVALID;
    if (g.algo == AR_ALGO_TWOSHOT)
        return AR_ERR_INVALID;
    if (!g.cap_ready && (rc = compute_capacity()) != AR_OK)
        return rc;
    const size_t rows_cap = (size_t)g.capacity[ar::K_ONESHOT_ROWS_NORM][0][4] / g.n_ranks;
    if (p.kind == ar::K_ONESHOT_DIRECT_NORM && rows >= ar::ROWS_NORM_MIN_ROWS &&
        hidden <= ar::ROWS_NORM_MAX_HIDDEN && rows <= rows_cap) {
        p.kind = ar::K_ONESHOT_ROWS_NORM;
        p.threads = 1024;
        p.parts = (uint32_t)rows;
        p.slice = (uint32_t)slice_len(n, g.n_ranks);
        p.local = g.scope == AR_SCOPE_AUTO && g.placement_ok && p.parts % ar::XCDS == 0;
        p.rank_xcd = g.scope == AR_SCOPE_CROSS_XCD;
    } else {
        rc = plan_geometry(n, false, &p);
        if (rc != AR_OK)
            return rc;
    }
    if (g.step_rounds + p.rounds > ar::STEP_ROUNDS_MAX)
        return AR_ERR_INVALID;
    ar::NormLaunch L;
    memset(&L, 0, sizeof L);
    fill_launch(rank_bufs, out_h, n, epoch, p, &L.base);
    for (int r = 0; r < g.n_ranks; ++r)
        L.res[r] = residual[r];
    L.gamma = gamma;
    L.y = out_y;
    L.stats = g.stats;
    L.stats_stride = (uint32_t)g.stats_stride;
    L.hidden = (uint32_t)hidden;
    L.eps = eps;
    const uint32_t grid = p.parts * (uint32_t)g.n_ranks;
    if (debug_enabled())
        fprintf(stderr, "[ar] norm kind=%d rows=%zu hidden=%zu epoch=%u grid=%u threads=%u local=%d\n",
                p.kind, rows, hidden, epoch, grid, p.threads, (int)p.local);
    hipError_t e = ar::launch_norm(p.kind, p.local, L, p.threads, stream);
    if (e != hipSuccess)
        return hip_fail(e);
    g.last_epoch = epoch;
    g.step_rounds += p.rounds;
    return AR_OK;
}


// ---------------------------------------------------------------- no allocation
// The allocation-free variant of ar_allreduce (ar_allreduce_noalloc): the
// one-shot sentinel protocol with its inboxes in `scratch`, a file-scope
// device array (one per device, held until the process ends), so neither
// the call nor any set-up allocates.  Sentinel validity is in-band (an
// element is data once it is not 0xFFFF) and every consumed slot is re-armed
// within the call, so the inboxes need no flag sequence and are armed again
// when each call ends.  The array starts zeroed -- zero is data, not the
// sentinel -- so the first call on a device arms it first.
constexpr size_t NOALLOC_BYTES = size_t(4) << 20;          // [recv][send][2 buffers] x window
constexpr size_t NOALLOC_WINDOW_MAX = 64 * 1024;
constexpr int NOALLOC_MAX_DEVICES = 64;
static __device__ __align__(256) uint32_t scratch[NOALLOC_BYTES / 4];

struct NoAllocDevice {
    bool ready = false;                 // symbol address and device facts taken
    bool armed = false;                 // an eager arming has been enqueued
    uint32_t *ptr = nullptr;            // this device's copy of `scratch`
    uint32_t *ctl = nullptr;            // this device's control block (status record)
    int cu_count = 0;
    int per_cu[2] = {0, 0};             // resident workgroups per CU: <= 8 ranks, <= 16 ranks
};
NoAllocDevice g_na[NOALLOC_MAX_DEVICES];

// Window per (receiver, sender) pair and buffer: the largest multiple of
// 1 KiB with N^2 pairs x 2 buffers in the array, at most 64 KiB.
size_t noalloc_window(int n_ranks)
{
    const size_t w = NOALLOC_BYTES / (2 * (size_t)n_ranks * (size_t)n_ranks) / 1024 * 1024;
    return std::min(w, NOALLOC_WINDOW_MAX);
}

int noalloc_setup(int dev, NoAllocDevice *d)
{
    if (d->ready)
        return AR_OK;
    // with `dev` current: the array's address on this device (the host-side
    // name `scratch` is not a device address), the control block's, and the
    // facts the grid is sized with
    hipError_t e = hipGetSymbolAddress((void **)&d->ptr, HIP_SYMBOL(scratch));
    if (e == hipSuccess)
        e = ar::control_block(&d->ctl);
    if (e == hipSuccess)
        e = hipDeviceGetAttribute(&d->cu_count, hipDeviceAttributeMultiprocessorCount, dev);
    for (int i = 0; e == hipSuccess && i < 2; ++i)
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &d->per_cu[i], ar::kernel_for(ar::K_ONESHOT_SENTINEL, i == 0 ? 8 : 16, false, false, 0),
            512, 0);
    if (e != hipSuccess) {
        d->ptr = nullptr;
        return hip_fail(e);
    }
    d->ready = true;
    return AR_OK;
}

// Arms every inbox slot with the sentinel (a fill kernel, no memset node:
// capture-safe).  Marked armed only when enqueued eagerly: an arming
// captured into a graph runs only when that graph does.
int noalloc_arm(NoAllocDevice *d, hipStream_t stream)
{
    hipError_t e = ar::launch_fill(d->ptr, NOALLOC_BYTES / 4, ar::SENT_WORD, stream);
    if (e != hipSuccess)
        return hip_fail(e);
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    e = hipStreamIsCapturing(stream, &cs);
    if (e != hipSuccess)
        return hip_fail(e);
    d->armed = cs == hipStreamCaptureStatusNone;
    return AR_OK;
}

}  // namespace

extern "C" {

int ar_init(int n_ranks, size_t max_elems)
{
    if (g.live)
        return AR_ERR_STATE;
    if (n_ranks < 1 || n_ranks > AR_MAX_RANKS || max_elems == 0 || max_elems > MAX_ELEMS_LIMIT)
        return AR_ERR_INVALID;
    int env_algo = AR_ALGO_AUTO, env_proto = AR_PROTO_AUTO;
    uint32_t env_watchdog = DEFAULT_WATCHDOG_US;
    if (apply_env(&env_algo, &env_proto, &env_watchdog) != AR_OK)
        return AR_ERR_INVALID;
    hipError_t e = hipGetDevice(&g.device);
    if (e != hipSuccess)
        return hip_fail(e);
    e = hipDeviceGetAttribute(&g.cu_count, hipDeviceAttributeMultiprocessorCount, g.device);
    if (e != hipSuccess)
        return hip_fail(e);
    // the kernels' timers (watchdog budgets, start delays, call timestamps)
    // count the constant clock at 100 ticks per microsecond, the rate
    // MI355X reports; a device whose clock runs otherwise is refused
    e = hipDeviceGetAttribute(&g.wall_khz, hipDeviceAttributeWallClockRate, g.device);
    if (e != hipSuccess)
        return hip_fail(e);
    if (g.wall_khz != WALL_CLOCK_KHZ)
        return AR_ERR_INVALID;
    g.n_ranks = n_ranks;
    g.max_elems = round_up(max_elems, 8);
    const size_t me = g.max_elems;
    // staging windows: what the largest message needs in one round, at most
    // the fixed window sizes (larger messages take several rounds)
    auto window = [](size_t need, size_t quantum, size_t most) {
        return std::max(STAGE_WINDOW_MIN, std::min(round_up(need, quantum), most));
    };
    g.ll_stride = window(me * 4, STAGE_QUANTUM, STAGE_WINDOW_MAX);
    g.l128_stride = window((me + ar::L128_ELEMS - 1) / ar::L128_ELEMS * ar::L128_BYTES,
                           STAGE_QUANTUM_L128, STAGE_WINDOW_MAX);
    g.s1_stride = window(me * 2, STAGE_QUANTUM, STAGE_INBOX_MAX);
    g.s2_stride = window(slice_len(me, n_ranks) * 2, STAGE_QUANTUM, STAGE_INBOX_MAX);
    g.window = 0;
    g.stats_stride = (me + ar::NORM_BLOCK_ELEMS - 1) / ar::NORM_BLOCK_ELEMS;
    g.acc_stride = round_up((me + ar::ATOM_LINE_ELEMS - 1) / ar::ATOM_LINE_ELEMS * 128, 256);
    // the kernels skip a load or store by sending it to offset ar::OFF_NONE,
    // which must lie past the end of every input and output descriptor (the
    // largest is all N output copies in binary32: the binding size limit);
    // the staging windows are bounded far below it, and the atomic lines
    // (128 bytes per 31 elements, two buffers) stay below it too
    if (me * (size_t)n_ranks * 4 > (size_t)ar::OFF_NONE || acc_bytes() > (size_t)ar::OFF_NONE ||
        ll_bytes() > REGION_LIMIT || l128_bytes() > REGION_LIMIT || s1_bytes() > REGION_LIMIT ||
        s2_bytes() > REGION_LIMIT)
        return AR_ERR_INVALID;
    int rc;
    if ((rc = alloc(&g.ll, ll_bytes())) != AR_OK ||
        (rc = alloc(&g.l128, l128_bytes())) != AR_OK ||
        (rc = alloc(&g.s1, s1_bytes())) != AR_OK ||
        (rc = alloc(&g.srs, s2_bytes())) != AR_OK ||
        (rc = alloc(&g.sag, s2_bytes())) != AR_OK ||
        (rc = (ar::control_block(&g.ctl) == hipSuccess ? AR_OK : AR_ERR_HIP)) != AR_OK ||
        (rc = alloc((char **)&g.done, done_words() * 4)) != AR_OK ||
        (rc = alloc((char **)&g.stats, stats_bytes())) != AR_OK ||
        (rc = alloc(&g.acc, acc_bytes())) != AR_OK) {
        free_all();
        return rc;
    }
    e = rearm(0);
    if (e == hipSuccess)
        e = verify_placement(&g.placement_ok);
    if (e == hipSuccess)
        e = hipDeviceSynchronize();
    if (e != hipSuccess) {
        free_all();
        return hip_fail(e);
    }
    g.algo = env_algo; g.proto = env_proto;
    g.wgs_per_rank = 0; g.threads = 0;
    g.scope = AR_SCOPE_AUTO;
    g.watchdog_us = env_watchdog;
    g.delays = nullptr; g.delay_rows = 0;
    g.ts = nullptr; g.ts_slots = 0; g.ts_stride = 0; g.ts_phases = false;
    g.last_epoch = 0;
    g.step_rounds = 0;
    g.cap_ready = false;
    g.live = true;
    rc = compute_capacity();
    if (rc != AR_OK) {
        g.live = false;
        free_all();
        return rc;
    }
    if (debug_enabled())
        fprintf(stderr, "[ar] init N=%d max_elems=%zu CUs=%d staging=%zu B\n", n_ranks, me,
                g.cu_count, ll_bytes() + l128_bytes() + s1_bytes() + 2 * s2_bytes());
    return AR_OK;
}

int ar_destroy(void)
{
    if (!g.live)
        return AR_ERR_NOT_INIT;
    free_all();
    g.live = false;
    return AR_OK;
}

int ar_allreduce(const void *const *rank_bufs, void *out, size_t n, uint32_t epoch,
                 hipStream_t stream)
{
    return do_allreduce(rank_bufs, out, n, epoch, stream, false);
}

int ar_allreduce_add_rmsnorm(const void *const *rank_bufs, const void *const *residual,
                             const void *gamma, float eps, void *out_h, void *out_y, size_t rows,
                             size_t hidden, uint32_t epoch, hipStream_t stream)
{
    return do_allreduce_norm(rank_bufs, residual, gamma, eps, out_h, out_y, rows, hidden, epoch,
                             stream);
}

int ar_add_rmsnorm(const void *a, const void *const *residual, const void *gamma, float eps,
                   void *out_h, void *out_y, size_t rows, size_t hidden, hipStream_t stream)
{
    if (!g.live)
        return AR_ERR_NOT_INIT;
    size_t n = 0;
    const void *src[1] = {a};
    int rc = check_norm(src, 1, residual, gamma, eps, out_h, out_y, rows, hidden, &n);
    if (rc != AR_OK)
        return rc;
    hipError_t e = ar::launch_add_rmsnorm(a, residual, gamma, eps, out_h, out_y,
                                          (uint32_t)g.n_ranks, (uint32_t)rows, (uint32_t)hidden,
                                          stream);
    if (e != hipSuccess)
        return hip_fail(e);
    return AR_OK;
}

int ar_allreduce_f32_debug(const void *const *rank_bufs, float *out_f32, size_t n, uint32_t epoch,
                           hipStream_t stream)
{
    return do_allreduce(rank_bufs, out_f32, n, epoch, stream, true);
}

int ar_set_options(int algo, int proto)
{
    if (!g.live)
        return AR_ERR_NOT_INIT;
    if (algo < AR_ALGO_AUTO || algo > AR_ALGO_TWOSHOT)
        return AR_ERR_INVALID;
    if (proto < AR_PROTO_AUTO || proto > AR_PROTO_ATOMIC)
        return AR_ERR_INVALID;
    if (algo == AR_ALGO_TWOSHOT && proto == AR_PROTO_LL)
        return AR_ERR_INVALID;
    if (algo == AR_ALGO_ONESHOT && proto == AR_PROTO_ATOMIC)
        return AR_ERR_INVALID;
    g.algo = algo;
    g.proto = proto;
    return AR_OK;
}

int ar_set_launch(int wgs_per_rank, int threads)
{
    if (!g.live)
        return AR_ERR_NOT_INIT;
    if (wgs_per_rank < 0 || !(threads == 0 || threads == 64 || threads == 128 || threads == 256))
        return AR_ERR_INVALID;
    g.wgs_per_rank = wgs_per_rank;
    g.threads = threads;
    return AR_OK;
}

int ar_set_scope(int scope)
{
    if (!g.live)
        return AR_ERR_NOT_INIT;
    if (scope != AR_SCOPE_AUTO && scope != AR_SCOPE_DEVICE && scope != AR_SCOPE_CROSS_XCD)
        return AR_ERR_INVALID;
    g.scope = scope;
    return AR_OK;
}

int ar_set_staging(size_t window_bytes)
{
    if (!g.live)
        return AR_ERR_NOT_INIT;
    if (window_bytes != 0 && (window_bytes < STAGE_WINDOW_MIN || window_bytes % STAGE_ROUND_BYTES))
        return AR_ERR_INVALID;
    g.window = window_bytes;            // each call plans its own rounds: any time
    return AR_OK;
}

int ar_set_watchdog(uint32_t budget_us)
{
    if (!g.live)
        return AR_ERR_NOT_INIT;
    g.watchdog_us = budget_us ? budget_us : DEFAULT_WATCHDOG_US;   // 0: the built-in default
    return AR_OK;
}

int ar_step_end(hipStream_t stream)
{
    if (!g.live)
        return AR_ERR_NOT_INIT;
    if (g.last_epoch > 0) {
        hipError_t e = ar::launch_step_end(g.ctl, g.last_epoch, (uint32_t)g.step_rounds, g.ll,
                                           ll_bytes(), g.l128, l128_bytes(), g.done, g.stats,
                                           stats_bytes(), stream);
        if (e != hipSuccess)
            return hip_fail(e);
    }
    g.last_epoch = 0;
    g.step_rounds = 0;
    return AR_OK;
}

int ar_set_sequence(uint32_t seq, hipStream_t stream)
{
    if (!g.live)
        return AR_ERR_NOT_INIT;
    if (g.last_epoch != 0)
        return AR_ERR_STATE;            // only between steps
    if (seq > ar::SEQ_WRAP)
        return AR_ERR_INVALID;
    hipError_t e = ar::launch_set_seq(g.ctl, seq, stream);
    if (e != hipSuccess)
        return hip_fail(e);
    return AR_OK;
}

int ar_set_delays(const uint32_t *dev_ns, size_t calls)
{
    if (!g.live)
        return AR_ERR_NOT_INIT;
    if (dev_ns != nullptr && (calls == 0 || calls > 0xFFFFFFFFu / (size_t)g.n_ranks / 4))
        return AR_ERR_INVALID;
    g.delays = dev_ns;
    g.delay_rows = dev_ns ? calls : 0;
    return AR_OK;
}

int ar_set_timestamps(uint64_t *dev_ts, size_t slots, size_t records_per_slot, int phases)
{
    if (!g.live)
        return AR_ERR_NOT_INIT;
    if (dev_ts != nullptr && (slots == 0 || slots > 0xFFFFFFFFu || records_per_slot == 0 ||
                              records_per_slot > 0xFFFFFFFFu ||
                              slots > ((size_t)1 << 40) / records_per_slot))
        return AR_ERR_INVALID;
    g.ts = dev_ts;
    g.ts_slots = dev_ts ? slots : 0;
    g.ts_stride = dev_ts ? records_per_slot : 0;
    g.ts_phases = dev_ts != nullptr && phases != 0;
    return AR_OK;
}

int ar_get_status(uint32_t out[4])
{
    if (!g.live)
        return AR_ERR_NOT_INIT;
    if (out == nullptr)
        return AR_ERR_INVALID;
    hipError_t e = hipDeviceSynchronize();
    if (e != hipSuccess)
        return hip_fail(e);
    e = hipMemcpy(out, g.ctl + ar::CTL_STATUS, 16, hipMemcpyDeviceToHost);
    if (e != hipSuccess)
        return hip_fail(e);
    return out[0] == ar::STATUS_TIMEOUT ? AR_ERR_TIMEOUT : AR_OK;
}

int ar_allreduce_noalloc(const void *const *rank_bufs, void *out, size_t n, int n_ranks,
                         hipStream_t stream)
{
    if (n_ranks < 1 || n_ranks > AR_MAX_RANKS)
        return AR_ERR_INVALID;
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return hip_fail(e);
    if (dev < 0 || dev >= NOALLOC_MAX_DEVICES)
        return AR_ERR_INVALID;
    NoAllocDevice &d = g_na[dev];
    int rc = noalloc_setup(dev, &d);
    if (rc != AR_OK)
        return rc;
    if (n == 0)                          // re-arm (after a call that a watchdog ended)
        return noalloc_arm(&d, stream);
    // sizes: 8-element vectors; all N output copies below 2^31 bytes (the
    // kernels' skipped-access offset lies past every descriptor)
    if (rank_bufs == nullptr || out == nullptr || n % 8 != 0 ||
        n * (size_t)n_ranks * 2 > (size_t)ar::OFF_NONE)
        return AR_ERR_INVALID;
    const uintptr_t o = (uintptr_t)out, o_end = o + 2 * n * (size_t)n_ranks;
    if (o % 16)
        return AR_ERR_INVALID;
    for (int r = 0; r < n_ranks; ++r) {
        const uintptr_t b = (uintptr_t)rank_bufs[r];
        if (b == 0 || b % 16 || (b < o_end && o < b + 2 * n))
            return AR_ERR_INVALID;
    }
    if (!d.armed && (rc = noalloc_arm(&d, stream)) != AR_OK)
        return rc;
    // geometry: 64 chunks of 8 elements per workgroup and round, one round of
    // every part within the window, the grid resident at once
    const size_t win = noalloc_window(n_ranks);
    const uint64_t chunks = n / 8;
    uint64_t cap = (uint64_t)d.per_cu[n_ranks <= 8 ? 0 : 1] * (uint64_t)d.cu_count / (uint64_t)n_ranks;
    cap = std::min<uint64_t>(cap, win / STAGE_ROUND_BYTES);
    if (cap == 0)
        return AR_ERR_INVALID;
    uint64_t parts = std::max<uint64_t>(1, ceil_div(chunks, 64));
    const uint64_t up = round_up(parts, ar::XCDS);
    parts = up <= cap ? up : (cap >= ar::XCDS ? cap / ar::XCDS * ar::XCDS : cap);
    parts = std::min(parts, cap);
    Launch a;
    memset(&a, 0, sizeof a);
    for (int r = 0; r < n_ranks; ++r)
        a.in[r] = rank_bufs[r];
    a.out = out;
    a.s1 = (char *)d.ptr;
    a.s1_stride = (uint32_t)win;
    a.ctl = d.ctl;                      // status record: the one ar_get_status reads
    a.n = (uint32_t)n;
    a.n_ranks = (uint32_t)n_ranks;
    a.epoch = 1;                        // buffer parity and records only: no flags
    a.parts = (uint32_t)parts;
    a.slice = (uint32_t)slice_len(n, n_ranks);
    a.xshift = parts % ar::XCDS == 0 ? 3u : 0u;
    a.watchdog_ticks = DEFAULT_WATCHDOG_US * 100u;
    e = ar::launch_ar(ar::K_ONESHOT_SENTINEL, false, false, 0, a, 512, stream);
    if (e != hipSuccess)
        return hip_fail(e);
    return AR_OK;
}

int ar_reset(hipStream_t stream)
{
    if (!g.live)
        return AR_ERR_NOT_INIT;
    hipError_t e = rearm(stream);
    if (e != hipSuccess)
        return hip_fail(e);
    g.last_epoch = 0;
    g.step_rounds = 0;
    return AR_OK;
}

const char *ar_strerror(int status)
{
    switch (status) {
    case AR_OK: return "ok";
    case AR_ERR_INVALID: return "invalid argument";
    case AR_ERR_NOT_INIT: return "library not initialised";
    case AR_ERR_STATE: return "invalid call order or state";
    case AR_ERR_OOM: return "device out of memory";
    case AR_ERR_HIP: return "HIP runtime error";
    case AR_ERR_TIMEOUT: return "device poll exceeded the watchdog";
    default: return "unknown status";
    }
}

int ar_last_hip_error(void) { return g_last_hip; }

long long ar_query(int key, size_t n)
{
    if (!g.live)
        return AR_ERR_NOT_INIT;
    Plan p;
    switch (key) {
    case 0: return g.n_ranks;
    case 1: return (long long)g.max_elems;
    case 2:
    case 3:
    case 4:
    case 5: {
        if (n == 0 || n > g.max_elems || n % 8)
            return AR_ERR_INVALID;
        int rc = make_plan(n, false, &p);
        if (rc != AR_OK)
            return rc;
        if (key == 2)
            return (p.kind == ar::K_TWOSHOT_LL128 || p.kind == ar::K_TWOSHOT_SENTINEL ||
                    p.kind == ar::K_TWOSHOT_DIRECT || p.kind == ar::K_TWOSHOT_BARRIER ||
                    p.kind == ar::K_TWOSHOT_ATOMIC)
                       ? AR_ALGO_TWOSHOT : AR_ALGO_ONESHOT;
        if (key == 3) {
            switch (p.kind) {
            case ar::K_ONESHOT_LL: return AR_PROTO_LL;
            case ar::K_ONESHOT_DIRECT:
            case ar::K_TWOSHOT_DIRECT: return AR_PROTO_DIRECT;
            case ar::K_ONESHOT_BARRIER:
            case ar::K_TWOSHOT_BARRIER: return AR_PROTO_BARRIER;
            case ar::K_ONESHOT_SENTINEL:
            case ar::K_TWOSHOT_SENTINEL: return AR_PROTO_SENTINEL;
            case ar::K_TWOSHOT_ATOMIC: return AR_PROTO_ATOMIC;
            default: return AR_PROTO_LL128;
            }
        }
        if (key == 4) return (long long)p.parts * g.n_ranks;
        return p.threads;
    }
    case 6: {
        int kind;
        if (n == 0 || choose_kind(n, &kind) != AR_OK) return AR_ERR_INVALID;
        if (!g.cap_ready && compute_capacity() != AR_OK) return AR_ERR_HIP;
        return g.capacity[kind][0][2];
    }
    case 7: return g.last_epoch;
    case 8: {
        if (n == 0 || n > g.max_elems || n % 8)
            return AR_ERR_INVALID;
        int rc = make_plan(n, false, &p);
        return rc != AR_OK ? rc : (p.local ? 1 : 0);
    }
    case 9: return g.placement_ok ? 1 : 0;
    case 10: return g.wall_khz;
    case 11: return g.cu_count;
    case 12: {
        if (n == 0 || n > g.max_elems || n % 8)
            return AR_ERR_INVALID;
        int rc = make_plan(n, false, &p);
        return rc != AR_OK ? rc : (long long)p.rounds;
    }
    case 13: return (long long)g.step_rounds;
    case 16: {
        if (n == 0 || n > g.max_elems || n % 8)
            return AR_ERR_INVALID;
        int rc = make_plan(n, false, &p);
        return rc != AR_OK ? rc : (p.rank_xcd || p.parts % ar::XCDS != 0 ? 1 : 0);
    }
    case 15: {
        int kind;
        if (n == 0 || choose_kind(n, &kind) != AR_OK) return AR_ERR_INVALID;
        return (long long)window_of(kind);
    }
    case 14: {
        uint32_t w[2] = {0, 0};
        hipError_t e = hipDeviceSynchronize();
        if (e == hipSuccess)
            e = hipMemcpy(w, g.ctl + ar::CTL_SEQ, 8, hipMemcpyDeviceToHost);
        if (e != hipSuccess)
            return hip_fail(e);
        return n == 0 ? (long long)w[0] : (long long)w[1];
    }
    default: return AR_ERR_INVALID;
    }
}

}  // extern "C"
