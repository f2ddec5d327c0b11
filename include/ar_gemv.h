/*
 * ar_gemv.h -- the decode projection that produces the AllReduce input, for
 *              the compute/communication overlap harness (MI355X, gfx950).
 *
 * In a tensor-parallel decode layer each rank multiplies its weight shard by
 * its share of the activation; the row-parallel layers end in an AllReduce
 * that sums the per-rank partial products ("vLLM 分布式推理核心" page,
 * section 一: two AllReduces per layer at TP = 8, hidden 8192).  This entry
 * point computes those partial products for all emulated ranks:
 *
 *   y_r[m] = bf16_rne( sum over k of W_r[m][k] * x_r[k] )   r = 0..n_ranks-1
 *
 * accumulated in binary32 (each wave owns four consecutive rows; per row a
 * lane sums its 8-element chunks in order, then the 64 lanes combine in a
 * fixed butterfly), so the
 * result is deterministic but, unlike the AllReduce, not bit-identical to a
 * sequential sum; the tests hold it to the binary32 error bound of that
 * summation order.  It is not part of the AllReduce path; the overlap
 * harness runs it on a compute stream beside the AllReduce.
 *
 * Conventions as in ar.h: int status (AR_OK or a negative ar_status code),
 * plain device pointers owned by the caller, asynchronous on `stream`, no
 * allocation (capture-safe).  It needs no ar_init.
 */
#ifndef TPDC_AR_GEMV_H
#define TPDC_AR_GEMV_H

#include <stddef.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * ar_gemv_bf16 -- y_r = W_r x_r for every rank r.
 *   W:  host array of n_ranks device pointers to bf16 [M][K] (row-major),
 *       16-byte aligned;
 *   x:  host array of n_ranks device pointers to bf16 [K], 16-byte aligned;
 *   y:  host array of n_ranks device pointers to bf16 [M] (outputs; must
 *       not overlap W or x), 2-byte aligned;
 *   M >= 1 rows; K >= 8 with K % 8 == 0, K <= 2^28 and M*K*2 < 2^32;
 *   1 <= n_ranks <= 16;
 *   max_workgroups: cap on the grid (256-thread workgroups, 4 rows each,
 *       rows beyond the grid are processed grid-stride); 0 = automatic
 *       (up to 8192).  A cap leaves CUs free for a concurrent AllReduce.
 * Returns AR_ERR_INVALID for arguments outside this contract, AR_ERR_HIP if
 * the launch fails, else AR_OK.
 */
int ar_gemv_bf16(const void *const *W, const void *const *x, void *const *y, size_t M, size_t K,
                 int n_ranks, int max_workgroups, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif
