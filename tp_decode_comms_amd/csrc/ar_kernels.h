// ar_kernels.h -- host-side entry points into the kernels (internal).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ar {

struct Launch;
struct NormLaunch;

// residual add + RMS norm: the row length is a multiple of the 256-element
// block of one partial sum, at most 65536
constexpr size_t NORM_BLOCK_ELEMS = 256;
constexpr size_t NORM_HIDDEN_LIMIT = 65536;
// the row-wise fused kernel: one 16-wave workgroup per (rank, row), for at
// least this many rows of at most ROWS_NORM_MAX_HIDDEN elements
constexpr size_t ROWS_NORM_MIN_ROWS = 8;
constexpr size_t ROWS_NORM_MAX_HIDDEN = 8192;
// two-shot DIRECT: 8-element chunks each lane reduces per round
constexpr uint32_t TWOSHOT_DIRECT_CHUNKS = 2;
// atomic lines: 128 bytes = a 4-byte counter and 31 binary32 sums
constexpr size_t ATOM_LINE_ELEMS = 31;

enum KernelKind {
    K_ONESHOT_LL = 0,
    K_ONESHOT_SENTINEL = 1,
    K_ONESHOT_DIRECT = 2,
    K_ONESHOT_LL128 = 3,
    K_TWOSHOT_LL128 = 4,
    K_TWOSHOT_SENTINEL = 5,
    K_TWOSHOT_DIRECT = 6,
    K_ONESHOT_BARRIER = 7,
    K_TWOSHOT_BARRIER = 8,
    K_ONESHOT_LL_NORM = 9,      // one-shot LL + residual add + RMS norm (bf16 only)
    K_TWOSHOT_ATOMIC = 10,      // atomic lines (arrival-order sums: not bit-exact)
    K_ONESHOT_DIRECT_NORM = 11, // one-shot DIRECT + residual add + RMS norm (bf16 only)
    K_ONESHOT_ROWS_NORM = 12,   // the same, one workgroup per (rank, row)
    K_COUNT = 13
};

// device function of a kernel kind for n_ranks (<= 8 or <= 16 instantiation);
// local selects the XCD-local coherence scope (bf16 kernels only)
// gw: line groups per batch of the LL128 kinds (1, 2 or 4; 0 = the largest
// available), ignored by the others
// hooks: the measurement and test hooks built in (0 none, 1 start records,
// 2 all: start delays, start or phase records; bf16 -- the fp32 debug
// kernels always have all)
const void *kernel_for(int kind, int n_ranks, bool f32, bool local, int gw, int hooks = 0);

// grid (2^xshift, N, parts >> xshift) from the launch record (parts must be a
// multiple of 2^xshift)
hipError_t launch_ar(int kind, bool f32, bool local, int gw, const Launch &a, uint32_t threads,
                     hipStream_t stream);
// the fused AllReduce + residual add + RMS norm (kind K_ONESHOT_LL_NORM,
// K_ONESHOT_DIRECT_NORM or K_ONESHOT_ROWS_NORM)
hipError_t launch_norm(int kind, bool local, const NormLaunch &L, uint32_t threads,
                       hipStream_t stream);
// stand-alone residual add + RMS norm of an AllReduce result: one workgroup
// of 1024 threads per (rank, row)
hipError_t launch_add_rmsnorm(const void *a, const void *const *res, const void *gamma, float eps,
                              void *h, void *y, uint32_t n_ranks, uint32_t rows, uint32_t hidden,
                              hipStream_t stream);
// out[b] = XCD index of the workgroup with linear index b = x + gx (y + gy z),
// over a gx x gy x gz grid
hipError_t launch_xcc_map(uint32_t *out, uint32_t gx, uint32_t gy, uint32_t gz, uint32_t threads,
                          hipStream_t stream);
hipError_t launch_step_end(uint32_t *ctl, uint32_t calls, uint32_t rounds, char *ll,
                           size_t ll_bytes, char *l128, size_t l128_bytes, uint32_t *done,
                           uint32_t *stats, size_t stats_bytes, hipStream_t stream);
hipError_t launch_set_seq(uint32_t *ctl, uint32_t seq, hipStream_t stream);
hipError_t launch_fill(uint32_t *p, size_t words, uint32_t value, hipStream_t stream);
// device address of the control block (CTL_WORDS words) on the current device
hipError_t control_block(uint32_t **p);

}  // namespace ar
