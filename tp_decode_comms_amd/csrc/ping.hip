// ping.hip -- the flag hop between two workgroups (include/ar_ping.h): the
// latency floor that the small AllReduce calls are read against, beside the
// launch floor of a graph node.
//
// Two single-lane waves bounce a counter through two flag words with the
// same store and poll policies as the AllReduce kernels: XCD-local (both
// workgroups on one XCD, stores and polls coherent in its L2) or across XCDs
// (device scope).  Workgroup A stores value v and waits for B's copy of v; B
// waits for A's v and stores it back.  A times the whole exchange on the
// constant 100 MHz clock: one way is that time / (2 rounds).  Every wait is
// bounded by a clock budget, so the kernel ends whether or not the partner
// ever answers.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/ar.h"
#include "../../include/ar_ping.h"
#include "ar_proto.h"

namespace ar {

// A's word at byte 0, B's at byte 128: each on a 128-byte line of its own.
// The values only grow from call to call (the host hands each call the base
// after the previous call's last value), so the words are never cleared.
__device__ __align__(256) uint32_t ping_words[64];

constexpr uint32_t PING_MAX_ROUNDS = 1u << 20;
constexpr uint32_t PING_BUDGET_TICKS = 20000000u;   // 200 ms of the 100 MHz clock

// Grid: XCD-local, 9 one-wave workgroups (blocks 0 and 8 share an XCD under
// the round-robin dispatch, whatever XCD block 0 starts on; blocks 1..7 exit
// at once); across XCDs, 2 (blocks 0 and 1, on neighbouring XCDs).  out (5 words of 8 bytes): ticks, A's status, A's XCD, B's XCD,
// B's status; status 1 = a wait ran out of budget.
template <bool LOCAL>
__global__ __launch_bounds__(64) void k_ping(uint32_t base, uint32_t rounds, uint32_t partner, void *out)
{
    const bool is_a = blockIdx.x == 0u;
    if ((!is_a && blockIdx.x != partner) || threadIdx.x != 0u)
        return;
    const __amdgpu_buffer_rsrc_t w = rsrc(ping_words, sizeof(ping_words));
    const uint32_t mine = is_a ? 0u : 128u, theirs = is_a ? 128u : 0u;
    const uint64_t t0 = clock100();
    uint32_t status = 0;
    for (uint32_t i = 1; i <= rounds; ++i) {
        const uint32_t v = base + i;
        if (is_a)
            st4<Pol<LOCAL>::ST>(v, w, mine);
        // the budget is checked every 16th poll: a clock read is a scalar
        // memory instruction, and between two polls it would lengthen the hop
        uint32_t it = 0;
        while ((int32_t)(ld4<Pol<LOCAL>::LD>(w, theirs) - v) < 0) {
            if ((++it & 15u) == 0u && clock100() - t0 > PING_BUDGET_TICKS) {
                status = 1;
                break;
            }
        }
        if (status != 0u)
            break;
        if (!is_a)
            st4<Pol<LOCAL>::ST>(v, w, mine);
    }
    const uint64_t ticks = clock100() - t0;
    const __amdgpu_buffer_rsrc_t o = rsrc(out, 5u * 8u);
    if (is_a) {
        st4<CP_PLAIN>((uint32_t)ticks, o, 0u);
        st4<CP_PLAIN>((uint32_t)(ticks >> 32), o, 4u);
        st4<CP_PLAIN>(status, o, 8u);
        st4<CP_PLAIN>(0u, o, 12u);
        st4<CP_PLAIN>(xcc_id(), o, 16u);
        st4<CP_PLAIN>(0u, o, 20u);
    } else {
        st4<CP_PLAIN>(xcc_id(), o, 24u);
        st4<CP_PLAIN>(0u, o, 28u);
        st4<CP_PLAIN>(status, o, 32u);
        st4<CP_PLAIN>(0u, o, 36u);
    }
}

}  // namespace ar

extern "C" int ar_flag_ping(uint32_t rounds, int cross_xcd, void *out, hipStream_t stream)
{
    // the next base per device: the values a call stores are base + 1 ..
    // base + rounds, above everything an earlier call left in the words
    static uint32_t next_base[64];
    if (rounds == 0 || rounds > ar::PING_MAX_ROUNDS || out == nullptr || (uintptr_t)out % 8 ||
        (cross_xcd != 0 && cross_xcd != 1))
        return AR_ERR_INVALID;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
        return AR_ERR_HIP;
    const uint32_t base = next_base[dev];
    next_base[dev] = base + rounds;
    if (cross_xcd)
        hipLaunchKernelGGL(ar::k_ping<false>, dim3(2), dim3(64), 0, stream, base, rounds, 1u, out);
    else
        hipLaunchKernelGGL(ar::k_ping<true>, dim3(9), dim3(64), 0, stream, base, rounds, 8u, out);
    return hipGetLastError() == hipSuccess ? AR_OK : AR_ERR_HIP;
}
