// gemv.hip -- the decode projection y_r = W_r x_r (bf16 in, binary32
// accumulate, bf16 out) of the compute/communication overlap harness.
//
// A batch-1 matrix-vector product streams the weights once: it is bound by
// HBM bandwidth, not by arithmetic, so it uses vector FMAs and no MFMA.  One
// wave per output row: lane l sums chunks l, l + 64, ... of the row (8
// elements, one 16-byte load of W and of x each), then the 64 lanes combine
// in a fixed xor butterfly.  x (K elements per rank) is re-read by every row
// of its rank and stays in the caches.
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

__global__ __launch_bounds__(256) void k_gemv(const GemvArgs a)
{
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t waves = gridDim.x * (blockDim.x >> 6);
    const uint32_t rows = a.M * a.n_ranks;
    const uint32_t chunks = a.K >> 3;
    for (uint32_t row = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6); row < rows;
         row += waves) {
        const uint32_t r = row / a.M, m = row % a.M;
        const __amdgpu_buffer_rsrc_t w = rsrc((const char *)a.W[r] + (size_t)m * a.K * 2u, a.K * 2u);
        const __amdgpu_buffer_rsrc_t xr = rsrc(a.x[r], a.K * 2u);
        float acc = 0.0f;
        for (uint32_t c = lane; c < chunks; c += 64u) {
            const u32x4 wv = ld16<CP_NT>(w, c * 16u);       // weights: streamed once
            const u32x4 xv = ld16<CP_PLAIN>(xr, c * 16u);
            acc = __builtin_fmaf(lo_f(wv.x), lo_f(xv.x), acc);
            acc = __builtin_fmaf(hi_f(wv.x), hi_f(xv.x), acc);
            acc = __builtin_fmaf(lo_f(wv.y), lo_f(xv.y), acc);
            acc = __builtin_fmaf(hi_f(wv.y), hi_f(xv.y), acc);
            acc = __builtin_fmaf(lo_f(wv.z), lo_f(xv.z), acc);
            acc = __builtin_fmaf(hi_f(wv.z), hi_f(xv.z), acc);
            acc = __builtin_fmaf(lo_f(wv.w), lo_f(xv.w), acc);
            acc = __builtin_fmaf(hi_f(wv.w), hi_f(xv.w), acc);
        }
#pragma unroll
        for (int off = 32; off > 0; off >>= 1)
            acc += __shfl_xor(acc, off, 64);
        if (lane == 0u) {
            const uint32_t two = pack_bf16(acc, 0.0f);
            ((uint16_t *)a.y[r])[m] = (uint16_t)(two & 0xFFFFu);
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
    if (M == 0 || K < 8 || K % 8 != 0 || M * K * 2 >= (size_t(1) << 32) ||
        M * (size_t)n_ranks >= (size_t(1) << 31))
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
    // 4 rows per workgroup, capped at a few waves per CU (grid-stride beyond)
    const size_t rows = M * (size_t)n_ranks;
    size_t blocks = (rows + 3) / 4;
    const size_t cap = max_workgroups > 0 ? (size_t)max_workgroups : 8192;
    if (blocks > cap)
        blocks = cap;
    hipLaunchKernelGGL(ar::k_gemv, dim3((unsigned)blocks), dim3(256), 0, stream, a);
    return hipGetLastError() == hipSuccess ? AR_OK : AR_ERR_HIP;
}
