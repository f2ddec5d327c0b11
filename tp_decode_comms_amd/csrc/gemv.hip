// gemv.hip -- the decode projection y_r = W_r x_r (bf16 in, binary32
// accumulate, bf16 out) of the compute/communication overlap harness.
//
// A batch-1 matrix-vector product streams the weights once: it is bound by
// HBM bandwidth, not by arithmetic, so it uses vector FMAs and no MFMA.  Each
// wave owns GEMV_ROWS consecutive rows of one rank.  Per row, lane l sums
// chunks l, l + 64, ... of the row (8 elements, one 16-byte load of W and of
// x each) in that order, then the 64 lanes combine in a fixed xor butterfly.
// The wave issues the weight loads of all its rows for two chunks per lane
// before the first FMA, so each lane keeps 2 x GEMV_ROWS weight loads in
// flight (one row at a time left the loads of a wave too few to cover the
// memory latency).  x (K elements per rank) is re-read by every row group of
// its rank and stays in the caches.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/ar.h"
#include "../../include/ar_gemv.h"
#include "ar_proto.h"

namespace ar {

struct GemvArgs {
    const void *W[MAX_RANKS];
    const void *x[MAX_RANKS];
    void *y[MAX_RANKS];
    uint32_t M, K, n_ranks;
};

constexpr uint32_t GEMV_ROWS = 4;

__device__ __forceinline__ float dot8(u32x4 w, u32x4 x, float acc)
{
    acc = __builtin_fmaf(lo_f(w.x), lo_f(x.x), acc);
    acc = __builtin_fmaf(hi_f(w.x), hi_f(x.x), acc);
    acc = __builtin_fmaf(lo_f(w.y), lo_f(x.y), acc);
    acc = __builtin_fmaf(hi_f(w.y), hi_f(x.y), acc);
    acc = __builtin_fmaf(lo_f(w.z), lo_f(x.z), acc);
    acc = __builtin_fmaf(hi_f(w.z), hi_f(x.z), acc);
    acc = __builtin_fmaf(lo_f(w.w), lo_f(x.w), acc);
    acc = __builtin_fmaf(hi_f(w.w), hi_f(x.w), acc);
    return acc;
}

__global__ __launch_bounds__(256) void k_gemv(const GemvArgs a)
{
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t waves = gridDim.x * (blockDim.x >> 6);
    const uint32_t per_rank = (a.M + GEMV_ROWS - 1u) / GEMV_ROWS;   // row groups of a rank
    const uint32_t groups = per_rank * a.n_ranks;
    const uint32_t chunks = a.K >> 3;
    const uint32_t rowb = a.K * 2u;
    for (uint32_t gi = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6); gi < groups;
         gi += waves) {
        const uint32_t r = gi / per_rank, m0 = (gi % per_rank) * GEMV_ROWS;
        const uint32_t nr = a.M - m0 < GEMV_ROWS ? a.M - m0 : GEMV_ROWS;   // rows present
        const __amdgpu_buffer_rsrc_t w = rsrc((const char *)a.W[r] + (size_t)m0 * rowb, nr * rowb);
        const __amdgpu_buffer_rsrc_t xr = rsrc(a.x[r], rowb);
        float acc[GEMV_ROWS];
#pragma unroll
        for (uint32_t k = 0; k < GEMV_ROWS; ++k)
            acc[k] = 0.0f;
        for (uint32_t c = lane; c < chunks; c += 128u) {
            // chunks c and c + 64 of every row; loads of absent rows and of a
            // chunk past the row end go past the descriptor's end (zeros, no
            // traffic) and their products are never added
            const bool two = c + 64u < chunks;
            u32x4 w0[GEMV_ROWS], w1[GEMV_ROWS];
#pragma unroll
            for (uint32_t k = 0; k < GEMV_ROWS; ++k) {
                w0[k] = ld16<CP_NT>(w, k < nr ? k * rowb + c * 16u : OFF_NONE);   // streamed once
                w1[k] = ld16<CP_NT>(w, k < nr && two ? k * rowb + (c + 64u) * 16u : OFF_NONE);
            }
            const u32x4 x0 = ld16<CP_PLAIN>(xr, c * 16u);
            const u32x4 x1 = ld16<CP_PLAIN>(xr, two ? (c + 64u) * 16u : OFF_NONE);
#pragma unroll
            for (uint32_t k = 0; k < GEMV_ROWS; ++k)
                acc[k] = dot8(w0[k], x0, acc[k]);
            if (two) {
#pragma unroll
                for (uint32_t k = 0; k < GEMV_ROWS; ++k)
                    acc[k] = dot8(w1[k], x1, acc[k]);
            }
        }
        // every lane ends with each row's total; lane k writes row m0 + k
        float mine = 0.0f;
#pragma unroll
        for (uint32_t k = 0; k < GEMV_ROWS; ++k) {
            float v = acc[k];
#pragma unroll
            for (int off = 32; off > 0; off >>= 1)
                v += __shfl_xor(v, off, 64);
            if (lane == k)
                mine = v;
        }
        if (lane < nr) {
            const uint32_t packed = pack_bf16(mine, 0.0f);
            ((uint16_t *)a.y[r])[m0 + lane] = (uint16_t)(packed & 0xFFFFu);
        }
    }
}

}  // namespace ar

extern "C" int ar_gemv_bf16(const void *const *W, const void *const *x, void *const *y, size_t M,
                            size_t K, int n_ranks, int max_workgroups, hipStream_t stream)
{
    if (W == nullptr || x == nullptr || y == nullptr || n_ranks < 1 || n_ranks > ar::MAX_RANKS ||
        max_workgroups < 0)
        return AR_ERR_INVALID;
    // byte offsets within a row group's weights stay below 2^31 (the kernel
    // skips loads by sending them to offset 2^31, past the end)
    if (M == 0 || K < 8 || K % 8 != 0 || M * K * 2 >= (size_t(1) << 32) ||
        K * 2 * ar::GEMV_ROWS > (size_t)ar::OFF_NONE || M * (size_t)n_ranks >= (size_t(1) << 31))
        return AR_ERR_INVALID;
    ar::GemvArgs a;
    for (int r = 0; r < n_ranks; ++r) {
        const uintptr_t w = (uintptr_t)W[r], xv = (uintptr_t)x[r], yv = (uintptr_t)y[r];
        if (w == 0 || xv == 0 || yv == 0 || w % 16 || xv % 16 || yv % 2)
            return AR_ERR_INVALID;
        const uintptr_t y_end = yv + 2 * M;
        if ((yv < w + 2 * M * K && w < y_end) || (yv < xv + 2 * K && xv < y_end))
            return AR_ERR_INVALID;                  // output overlaps an input
        a.W[r] = W[r]; a.x[r] = x[r]; a.y[r] = y[r];
    }
    a.M = (uint32_t)M; a.K = (uint32_t)K; a.n_ranks = (uint32_t)n_ranks;
    // 4 waves per workgroup, each a group of GEMV_ROWS rows, capped at a few
    // waves per CU (grid-stride beyond)
    const size_t groups = (M + ar::GEMV_ROWS - 1) / ar::GEMV_ROWS * (size_t)n_ranks;
    size_t blocks = (groups + 3) / 4;
    const size_t cap = max_workgroups > 0 ? (size_t)max_workgroups : 8192;
    if (blocks > cap)
        blocks = cap;
    hipLaunchKernelGGL(ar::k_gemv, dim3((unsigned)blocks), dim3(256), 0, stream, a);
    return hipGetLastError() == hipSuccess ? AR_OK : AR_ERR_HIP;
}
