// norm.hip -- stand-alone residual add + RMS norm of an AllReduce result
// (the unfused form of the op after the AllReduce in a decode layer,
// "vLLM 分布式推理核心" page, section 一).  Arithmetic and summation order
// are those of norm_math.h, shared with the fused kernel, so both give the
// same bits.
#include <string.h>

#include "ar_kernels.h"
#include "norm_math.h"

namespace ar {

struct AddNormArgs {
    const void *a;                    // [N][n] AllReduce result
    const void *res[MAX_RANKS];       // rank residuals [n]
    const void *gamma;                // [hidden]
    void *h, *y;                      // [N][n]
    uint32_t rows, hidden;
    float eps;
};

constexpr int NORM_WAVES = 16;
constexpr int NORM_PER_WAVE = NORM_MAX_BLOCKS / NORM_WAVES;   // blocks a wave holds at most

// One workgroup of 16 waves per (rank, row): wave w takes the row's blocks
// w, w+16, ...; lane l holds elements [4l, 4l+4) of each; h stays in
// registers between the two passes, the block sums in LDS.
__global__ __launch_bounds__(1024) void k_add_rmsnorm(const AddNormArgs p)
{
    __shared__ float bsum[NORM_MAX_BLOCKS];
    __shared__ float rinv;
    const uint32_t rank = blockIdx.x / p.rows, row = blockIdx.x % p.rows;
    const uint32_t lane = threadIdx.x & 63u, wave = threadIdx.x >> 6;
    const uint32_t B = p.hidden / NORM_BLOCK;
    const uint32_t n = p.rows * p.hidden, nb = n * 2u;
    const __amdgpu_buffer_rsrc_t ar_ = rsrc((const char *)p.a + (size_t)rank * nb, nb);
    const __amdgpu_buffer_rsrc_t rr = rsrc(p.res[rank], nb);
    const __amdgpu_buffer_rsrc_t gr = rsrc(p.gamma, p.hidden * 2u);
    const __amdgpu_buffer_rsrc_t hr = rsrc((char *)p.h + (size_t)rank * nb, nb);
    const __amdgpu_buffer_rsrc_t yr = rsrc((char *)p.y + (size_t)rank * nb, nb);
    const uint32_t row0 = row * p.hidden;
    u32x2 hk[NORM_PER_WAVE];
#pragma unroll
    for (int k = 0; k < NORM_PER_WAVE; ++k) {
        const uint32_t j = wave + NORM_WAVES * k;
        if (j < B) {
            const uint32_t e = row0 + j * NORM_BLOCK + lane * 4u;
            const u32x2 hw = add_round4(ld8<CP_PLAIN>(ar_, e * 2u), ld8<CP_PLAIN>(rr, e * 2u));
            st8<CP_PLAIN>(hw, hr, e * 2u);
            hk[k] = hw;
            const float s = wave_sum(sumsq4(hw));
            if (lane == 0u)
                bsum[j] = s;
        }
    }
    __syncthreads();
    if (wave == 0u) {
        float part = lane < B ? bsum[lane] : 0.0f;
        for (uint32_t g0 = 64u; g0 < B; g0 += 64u) {
            const uint32_t j = g0 + lane;
            part = part + (j < B ? bsum[j] : 0.0f);
        }
        const float r = rms_inv(wave_sum(part), p.hidden, p.eps);
        if (lane == 0u)
            rinv = r;
    }
    __syncthreads();
    const float r = rinv;
#pragma unroll
    for (int k = 0; k < NORM_PER_WAVE; ++k) {
        const uint32_t j = wave + NORM_WAVES * k;
        if (j < B) {
            const uint32_t col = j * NORM_BLOCK + lane * 4u;
            const u32x2 gw = ld8<CP_PLAIN>(gr, col * 2u);
            st8<CP_PLAIN>(scale4(hk[k], gw, r), yr, (row0 + col) * 2u);
        }
    }
}

hipError_t launch_add_rmsnorm(const void *a, const void *const *res, const void *gamma, float eps,
                              void *h, void *y, uint32_t n_ranks, uint32_t rows, uint32_t hidden,
                              hipStream_t stream)
{
    if (n_ranks == 0 || n_ranks > (uint32_t)MAX_RANKS || rows == 0 || hidden == 0 ||
        hidden % NORM_BLOCK != 0 || hidden > NORM_MAX_HIDDEN)
        return hipErrorInvalidValue;
    AddNormArgs p;
    memset(&p, 0, sizeof p);
    p.a = a;
    for (uint32_t r = 0; r < n_ranks; ++r)
        p.res[r] = res[r];
    p.gamma = gamma;
    p.h = h;
    p.y = y;
    p.rows = rows;
    p.hidden = hidden;
    p.eps = eps;
    hipLaunchKernelGGL(k_add_rmsnorm, dim3(n_ranks * rows), dim3(1024), 0, stream, p);
    return hipGetLastError();
}

}  // namespace ar
