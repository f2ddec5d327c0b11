// copy.hip -- the plain device copy that serves as the bandwidth reference
// of the AllReduce's bandwidth-bound sizes (include/ar_copy.h).
//
// Launch shape of the two-shot data phase: 256-thread workgroups, lane i of
// the grid moves 16-byte vectors i + k*step (k = 0, 1; step = threads in the
// grid) per round, both loads issued before either store; plain loads,
// streaming stores (nothing is left dirty in the L2 for the launch boundary
// to write back).  A vector past the end is sent to OFF_NONE (zeros, no
// memory access) so every round issues the same straight run.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/ar.h"
#include "../../include/ar_copy.h"
#include "ar_proto.h"

namespace ar {

constexpr uint32_t COPY_THREADS = 256;
constexpr uint32_t COPY_MAX_WORKGROUPS = 512;

__global__ __launch_bounds__(256) void k_copy(const void *src, void *dst, uint32_t vecs)
{
    const uint32_t step = gridDim.x * COPY_THREADS;
    const __amdgpu_buffer_rsrc_t s = rsrc(src, vecs * 16u);
    const __amdgpu_buffer_rsrc_t d = rsrc(dst, vecs * 16u);
    for (uint32_t v = blockIdx.x * COPY_THREADS + threadIdx.x; v < vecs; v += 2u * step) {
        const uint32_t o0 = v * 16u;
        const uint32_t o1 = v + step < vecs ? (v + step) * 16u : OFF_NONE;
        const u32x4 x0 = ld16<CP_PLAIN>(s, o0);
        const u32x4 x1 = ld16<CP_PLAIN>(s, o1);
        st16<CP_NT>(x0, d, o0);
        st16<CP_NT>(x1, d, o1);
    }
}

}  // namespace ar

extern "C" int ar_copy(const void *src, void *dst, size_t bytes, hipStream_t stream)
{
    const uintptr_t s = (uintptr_t)src, d = (uintptr_t)dst;
    // offsets stay below OFF_NONE = 2^31, the skipped-access offset
    if (src == nullptr || dst == nullptr || s % 16 || d % 16 || bytes < 16 || bytes % 16 ||
        bytes > (size_t)ar::OFF_NONE - 16)
        return AR_ERR_INVALID;
    if (s < d + bytes && d < s + bytes)
        return AR_ERR_INVALID;                      // the ranges overlap
    const uint32_t vecs = (uint32_t)(bytes / 16);
    size_t blocks = (vecs + 2 * ar::COPY_THREADS - 1) / (2 * ar::COPY_THREADS);
    if (blocks > ar::COPY_MAX_WORKGROUPS)
        blocks = ar::COPY_MAX_WORKGROUPS;
    hipLaunchKernelGGL(ar::k_copy, dim3((unsigned)blocks), dim3(ar::COPY_THREADS), 0, stream, src,
                       dst, vecs);
    return hipGetLastError() == hipSuccess ? AR_OK : AR_ERR_HIP;
}
