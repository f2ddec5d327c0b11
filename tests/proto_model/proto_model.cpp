// proto_model.cpp -- host-thread model of the staged AllReduce protocols
// with fixed-size double-buffered staging (test infrastructure, CPU only).
//
// What it checks.  The double-buffer argument of the "Every Microsecond
// Counts" write-up (page "微秒必争…", section "破局之道：无屏障同步的四大核心
// 机制", item 3): a message larger than one exchange is sent in rounds through
// two buffers that alternate; receiving a peer's round-k data proves that
// peer has finished round k-1, so it permits overwriting the buffer that
// held round k-1.  Each thread plays one (rank, part) of the GPU kernels --
// or, with `waves`, one wave of a workgroup that splits its peers over
// several waves and meets at a barrier each round -- and walks the rounds of
// several consecutive calls (a join between calls stands for the launch
// boundary).  Staging is a window of parts x units elements per rank and
// buffer, reused every two rounds:
//   ll        8-byte units {payload, flag} (64-bit atomics: self-validating);
//   ll128     lines of plain payload words + an atomic flag stored with
//             release after the payload and polled with acquire, so
//             ThreadSanitizer sees any read of a line that a later round
//             overwrote without the permit;
//   sentinel  inboxes [recv][send] of 32-bit atomic words armed with the
//             sentinel; the receiver re-arms what it consumed before its next
//             round's pushes (release), which orders the re-arm before the
//             writer's reuse of the slot.
// Round j of a call whose first round has flag f uses flag f + j and buffer
// (f + j) & 1; f advances by the call's rounds.
//
// Planted mistakes (must make the run fail): single_buffer (one buffer),
// call_flag (one flag for every round of a call), eager_publish (round j+1
// published before round j is received), late_rearm (sentinel re-arm after
// the next round's pushes), no_barrier (waves of a workgroup do not meet
// before the next round's publish).
//
// usage: proto_model <ll|ll128|sentinel> <ranks> <parts> <units> <elems>
//                    <calls> <seed> <waves> [mutant]
// exit: 0 every output exact; 2 a wrong output; 3 a poll exceeded the
//       watchdog; 1 bad arguments.
#include <atomic>
#include <barrier>
#include <chrono>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <memory>
#include <random>
#include <string>
#include <thread>
#include <vector>

namespace {

constexpr uint32_t SENT = 0xFFFFFFFFu;

enum Proto { LL, LL128, SENTINEL };
enum Mutant { NONE, SINGLE_BUFFER, CALL_FLAG, EAGER_PUBLISH, LATE_REARM, NO_BARRIER };

struct Cfg {
    Proto proto;
    int N, P, U, M, calls, waves;
    uint32_t seed;
    Mutant mut;
};

struct Line {                       // one part's slice of an LL128 window
    std::vector<uint32_t> payload;  // plain words
    std::atomic<uint64_t> flag{0};
};

struct World {
    Cfg c;
    int W;                          // window: elements per rank and buffer
    std::vector<std::atomic<uint64_t>> ll;      // [rank][2][W]
    std::vector<std::unique_ptr<Line>> lines;   // [rank][2][part]
    std::vector<std::atomic<uint32_t>> inbox;   // [recv][send][2][W]
    std::vector<uint32_t> in;                   // [rank][M] of the current call
    std::vector<uint32_t> out;                  // [rank][M]
    std::atomic<int> fail{0};
    explicit World(const Cfg &cfg)
        : c(cfg), W(cfg.P * cfg.U), ll((size_t)cfg.N * 2 * W),
          inbox((size_t)cfg.N * cfg.N * 2 * W), in((size_t)cfg.N * cfg.M),
          out((size_t)cfg.N * cfg.M)
    {
        for (auto &u : ll) u.store(0);
        for (auto &u : inbox) u.store(SENT);
        for (int i = 0; i < cfg.N * 2 * cfg.P; ++i) {
            lines.emplace_back(new Line);
            lines.back()->payload.assign(cfg.U, 0u);
        }
    }
};

uint32_t value(uint32_t seed, int call, int r, int e)
{
    uint64_t x = seed * 0x9E3779B97F4A7C15ull ^ ((uint64_t)call << 40) ^ ((uint64_t)r << 32) ^ (uint64_t)e;
    x ^= x >> 33; x *= 0xff51afd7ed558ccdull; x ^= x >> 33; x *= 0xc4ceb9fe1a85ec53ull; x ^= x >> 33;
    uint32_t v = (uint32_t)x;
    return v == SENT ? 0x12345678u : v;          // data never equals the sentinel
}

struct Jitter {
    std::mt19937 g;
    explicit Jitter(uint32_t s) : g(s) {}
    void operator()()
    {
        uint32_t k = g() % 16;
        if (k == 0) std::this_thread::sleep_for(std::chrono::microseconds(g() % 50));
        else if (k < 6) std::this_thread::yield();
    }
};

// spin until ready() with a 2 s watchdog; false on expiry (or another failure)
template <typename F> bool poll(World &w, F ready)
{
    auto t0 = std::chrono::steady_clock::now();
    for (uint32_t it = 0;; ++it) {
        if (ready()) return true;
        if ((it & 1023u) == 0u) {
            if (w.fail.load(std::memory_order_relaxed)) return false;
            if (std::chrono::steady_clock::now() - t0 > std::chrono::seconds(2)) {
                w.fail.store(3);
                return false;
            }
            std::this_thread::yield();
        }
    }
}

// One (rank, part) -- or one wave `wv` of it -- walking the rounds of a call.
// `tile` is the workgroup's shared [rank][units] tile (the LDS tile of the
// GPU kernels): each wave stores the rows it received, wave 0 its own row,
// and wave 0 folds the tile once the waves have met.
void worker(World &w, int call, uint32_t f0, int R, int r, int p, int wv, std::barrier<> *bar,
            std::vector<uint32_t> *tile, uint32_t jseed)
{
    const Cfg &c = w.c;
    Jitter jit(jseed);
    const int N = c.N, U = c.U, W = w.W;
    auto flag_of = [&](int j) { return c.mut == CALL_FLAG ? f0 : f0 + (uint32_t)j; };
    auto buf_of = [&](int j) { return c.mut == SINGLE_BUFFER ? 0 : (int)((f0 + (uint32_t)j) & 1u); };
    auto elem = [&](int j, int u) { return (j * c.P + p) * U + u; };
    auto mine = [&](int s) { return s != r && s % c.waves == wv; };   // peers this wave receives
    auto publish = [&](int j) {
        if (wv != 0) return;                                           // wave 0 publishes
        const uint32_t f = flag_of(j);
        const int b = buf_of(j);
        for (int u = 0; u < U; ++u) {
            const int e = elem(j, u);
            const uint32_t v = e < c.M ? w.in[(size_t)r * c.M + e] : 0u;
            if (c.proto == LL) {
                w.ll[((size_t)r * 2 + b) * W + p * U + u].store(((uint64_t)f << 32) | v,
                                                                  std::memory_order_relaxed);
            } else if (c.proto == LL128) {
                w.lines[((size_t)r * 2 + b) * c.P + p]->payload[u] = v;
            } else {
                for (int q = 0; q < N; ++q)
                    if (q != r)
                        w.inbox[(((size_t)q * N + r) * 2 + b) * W + p * U + u].store(
                            v, std::memory_order_release);
            }
        }
        if (c.proto == LL128)
            w.lines[((size_t)r * 2 + b) * c.P + p]->flag.store(f, std::memory_order_release);
    };
    std::vector<uint32_t> &got = *tile;                  // [s * U + u]
    std::vector<int> rearm_pending;            // late_rearm: slots of the previous round
    auto rearm = [&](int j) {
        const int b = buf_of(j);
        for (int s = 0; s < N; ++s)
            if (mine(s))
                for (int u = 0; u < U; ++u)
                    w.inbox[(((size_t)r * N + s) * 2 + b) * W + p * U + u].store(
                        SENT, std::memory_order_relaxed);
    };
    const bool eager = c.mut == EAGER_PUBLISH;
    if (eager) publish(0);
    for (int j = 0; j < R; ++j) {
        const uint32_t f = flag_of(j);
        const int b = buf_of(j);
        jit();
        if (!eager) publish(j);
        else if (j + 1 < R) publish(j + 1);    // before round j is received: no permit
        if (c.mut == LATE_REARM && j > 0) rearm(j - 1);
        for (int k = 0; k < N; ++k) {
            const int s = (r + 1 + k) % N;     // peers in a rotating order
            if (!mine(s)) continue;
            jit();
            for (int u = 0; u < U; ++u) {
                bool ok;
                if (c.proto == LL) {
                    auto &cell = w.ll[((size_t)s * 2 + b) * W + p * U + u];
                    uint64_t x = 0;
                    ok = poll(w, [&] { x = cell.load(std::memory_order_relaxed); return (uint32_t)(x >> 32) == f; });
                    got[(size_t)s * U + u] = (uint32_t)x;
                } else if (c.proto == LL128) {
                    Line &ln = *w.lines[((size_t)s * 2 + b) * c.P + p];
                    ok = u > 0 || poll(w, [&] { return ln.flag.load(std::memory_order_acquire) == f; });
                    got[(size_t)s * U + u] = ln.payload[u];
                } else {
                    auto &cell = w.inbox[(((size_t)r * N + s) * 2 + b) * W + p * U + u];
                    uint32_t x = SENT;
                    ok = poll(w, [&] { x = cell.load(std::memory_order_acquire); return x != SENT; });
                    got[(size_t)s * U + u] = x;
                }
                if (!ok) return;
            }
        }
        if (c.proto == SENTINEL && c.mut != LATE_REARM) rearm(j);
        if (wv == 0) {
            for (int u = 0; u < U; ++u)
                got[(size_t)r * U + u] = elem(j, u) < c.M ? w.in[(size_t)r * c.M + elem(j, u)] : 0u;
        }
        const bool meet = bar != nullptr && c.mut != NO_BARRIER;
        if (meet) bar->arrive_and_wait();      // the tile is complete
        if (wv == 0) {                         // reduce in rank order
            for (int u = 0; u < U; ++u) {
                const int e = elem(j, u);
                if (e >= c.M) continue;
                uint32_t acc = 0;
                for (int s = 0; s < N; ++s) acc += got[(size_t)s * U + u];
                w.out[(size_t)r * c.M + e] = acc;
            }
        }
        if (meet) bar->arrive_and_wait();      // the tile is reused; next round's publish
    }
    if (c.mut == LATE_REARM && R > 0) rearm(R - 1);
}

}  // namespace

int main(int argc, char **argv)
{
    if (argc < 9) {
        fprintf(stderr, "usage: %s <ll|ll128|sentinel> ranks parts units elems calls seed waves [mutant]\n", argv[0]);
        return 1;
    }
    Cfg c{};
    std::string pr = argv[1];
    c.proto = pr == "ll" ? LL : pr == "ll128" ? LL128 : pr == "sentinel" ? SENTINEL : (Proto)-1;
    c.N = atoi(argv[2]); c.P = atoi(argv[3]); c.U = atoi(argv[4]); c.M = atoi(argv[5]);
    c.calls = atoi(argv[6]); c.seed = (uint32_t)strtoul(argv[7], nullptr, 10); c.waves = atoi(argv[8]);
    std::string m = argc > 9 ? argv[9] : "none";
    c.mut = m == "none" ? NONE : m == "single_buffer" ? SINGLE_BUFFER : m == "call_flag" ? CALL_FLAG
          : m == "eager_publish" ? EAGER_PUBLISH : m == "late_rearm" ? LATE_REARM
          : m == "no_barrier" ? NO_BARRIER : (Mutant)-1;
    if ((int)c.proto < 0 || (int)c.mut < 0 || c.N < 2 || c.P < 1 || c.U < 1 || c.M < 1 ||
        c.calls < 1 || c.waves < 1 || c.waves > c.N) {
        fprintf(stderr, "bad arguments\n");
        return 1;
    }
    World w(c);
    const int R = (c.M + w.W - 1) / w.W;
    uint32_t seq = 0;                    // flag of the next call's first round - 1
    for (int call = 0; call < c.calls; ++call) {
        for (int r = 0; r < c.N; ++r)
            for (int e = 0; e < c.M; ++e) w.in[(size_t)r * c.M + e] = value(c.seed, call, r, e);
        std::vector<std::thread> th;
        std::vector<std::unique_ptr<std::barrier<>>> bars;
        std::vector<std::unique_ptr<std::vector<uint32_t>>> tiles;
        for (int r = 0; r < c.N; ++r)
            for (int p = 0; p < c.P; ++p) {
                std::barrier<> *bar = nullptr;
                if (c.waves > 1) {
                    bars.emplace_back(new std::barrier<>(c.waves));
                    bar = bars.back().get();
                }
                tiles.emplace_back(new std::vector<uint32_t>((size_t)c.N * c.U, 0u));
                for (int wv = 0; wv < c.waves; ++wv)
                    th.emplace_back(worker, std::ref(w), call, seq + 1, R, r, p, wv, bar,
                                    tiles.back().get(),
                                    c.seed * 7919u + (uint32_t)((call * c.N + r) * c.P + p) * 31u + wv);
            }
        for (auto &t : th) t.join();                 // the launch boundary
        if (w.fail.load()) {
            fprintf(stderr, "call %d: a poll exceeded the watchdog\n", call);
            return 3;
        }
        for (int e = 0; e < c.M; ++e) {
            uint32_t want = 0;
            for (int r = 0; r < c.N; ++r) want += w.in[(size_t)r * c.M + e];
            for (int r = 0; r < c.N; ++r)
                if (w.out[(size_t)r * c.M + e] != want) {
                    fprintf(stderr, "call %d: rank %d element %d wrong\n", call, r, e);
                    return 2;
                }
        }
        seq += (uint32_t)R;
    }
    printf("ok: %s N=%d parts=%d units=%d elems=%d rounds=%d calls=%d waves=%d\n", argv[1], c.N,
           c.P, c.U, c.M, R, c.calls, c.waves);
    return 0;
}
