/*
 * ar_oracle.c -- plain CPU oracle for the fixed-order bf16 AllReduce.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg may load or call this file's library.  The
 * product path (the HIP library under tp_decode_comms_amd/) never does, and
 * this file shares no code, header, table or helper with it.
 *
 * What is computed, and where the pages define it:
 *
 *   - AllReduce sums every GPU's partial result and hands the full sum to
 *     every GPU: "Every Microsecond Counts" write-up ("微秒必争：英伟达与苏黎世联
 *     邦理工学院如何突破多GPU通信延迟极限"), section "张量并行与AllReduce".
 *   - recvReduce receives the N values and sums them in registers; the
 *     one-shot kernel reads its local value, broadcasts it, reduces all N
 *     values and writes the output: same page, section
 *     "统一原语与API设计：将算法转化为工程生产力".
 *   - The pages fix neither the summation order nor the precision.  Reading
 *     used here: one sequential left fold over ranks 0,1,...,N-1 in IEEE
 *     binary32 (round to nearest, ties to even), starting from the widened
 *     value of rank 0 (not from +0), then one round-to-nearest-even
 *     conversion of the binary32 sum to bfloat16.  Every output copy
 *     out[r] equals that one result.
 *
 *   res[i]    = bf16_rne( (((f32(x_0[i]) + f32(x_1[i])) + f32(x_2[i])) + ...) )
 *   out[r][i] = res[i]                for r = 0..N-1
 *
 * Build: plain C, -O2 -fno-fast-math, x86-64 SSE arithmetic under the
 * default MXCSR (no flush-to-zero, no denormals-are-zero), so binary32
 * subnormals are kept.  The optional thread count splits the element range
 * only; each element's fold order is unchanged.
 */
#include <stdint.h>
#include <stddef.h>
#include <string.h>
#include <math.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* bfloat16 is the upper half of an IEEE binary32 pattern: widening is exact. */
static float widen_bf16(uint16_t h)
{
    uint32_t bits = (uint32_t)h << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return f;
}

/*
 * binary32 -> bfloat16, round to nearest, ties to even.
 *
 * For a finite binary32 value the two bfloat16 neighbours in magnitude are
 * the truncated pattern `hi` and `hi + 1` (the next pattern up; above the
 * largest finite bfloat16 this is infinity, which is IEEE overflow under
 * round-to-nearest).  The dropped 16 bits `rest` decide: above half -> up,
 * below half -> down, exactly half -> the neighbour with an even last bit.
 * Sign-magnitude encoding makes the same rule hold for negative values.
 * NaN stays NaN with its sign; the quiet bit is set so that a payload held
 * only in the dropped bits cannot turn into infinity.
 */
uint16_t oracle_f32_to_bf16(uint32_t f32_bits)
{
    uint32_t exponent = (f32_bits >> 23) & 0xFFu;
    uint32_t mantissa = f32_bits & 0x7FFFFFu;
    if (exponent == 0xFFu && mantissa != 0u)
        return (uint16_t)((f32_bits >> 16) | 0x0040u);
    uint32_t hi = f32_bits >> 16;
    uint32_t rest = f32_bits & 0xFFFFu;
    if (rest > 0x8000u || (rest == 0x8000u && (hi & 1u)))
        hi += 1u;
    return (uint16_t)hi;
}

/* Elementwise oracle_f32_to_bf16 over an array (for the exhaustive sweeps). */
void oracle_f32_to_bf16_array(const uint32_t *bits, size_t count, uint16_t *out)
{
    for (size_t i = 0; i < count; ++i)
        out[i] = oracle_f32_to_bf16(bits[i]);
}

/* binary32 sum of two binary32 patterns in the oracle's own arithmetic. */
uint32_t oracle_f32_add_bits(uint32_t a_bits, uint32_t b_bits)
{
    float a, b;
    memcpy(&a, &a_bits, sizeof a);
    memcpy(&b, &b_bits, sizeof b);
    float s = a + b;
    uint32_t out;
    memcpy(&out, &s, sizeof out);
    return out;
}

/* The binary32 accumulator of one element: the left fold over ranks. */
static float fold_element(const uint16_t *const *in, int n_ranks, size_t i)
{
    float acc = widen_bf16(in[0][i]);
    for (int r = 1; r < n_ranks; ++r)
        acc = acc + widen_bf16(in[r][i]);
    return acc;
}

/*
 * out is [n_ranks][n]: every rank's copy of the reduced vector.
 * threads <= 1 runs the plain sequential loop.
 */
void oracle_allreduce_bf16(const uint16_t *const *in, int n_ranks, size_t n,
                           uint16_t *out, int threads)
{
    if (n_ranks < 1 || n == 0)
        return;
#ifdef _OPENMP
#pragma omp parallel for schedule(static) num_threads(threads > 1 ? threads : 1) if (threads > 1)
#endif
    for (size_t i = 0; i < n; ++i) {
        float acc = fold_element(in, n_ranks, i);
        uint32_t bits;
        memcpy(&bits, &acc, sizeof bits);
        uint16_t res = oracle_f32_to_bf16(bits);
        for (int r = 0; r < n_ranks; ++r)
            out[(size_t)r * n + i] = res;
    }
}

/* The binary32 accumulators themselves, [n] (the fp32 result before rounding). */
void oracle_allreduce_f32(const uint16_t *const *in, int n_ranks, size_t n,
                          float *acc_out)
{
    if (n_ranks < 1)
        return;
    for (size_t i = 0; i < n; ++i)
        acc_out[i] = fold_element(in, n_ranks, i);
}

/* Threads the OpenMP runtime would use (1 when built without OpenMP). */
int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * Decode-step projection feeding the AllReduce (the overlap harness's
 * compute step).  In a tensor-parallel decode layer each rank multiplies its
 * weight shard by its share of the activation and the AllReduce sums the
 * per-rank partial products ("vLLM 分布式推理核心" page, section 一: the
 * row-parallel layers end in an AllReduce).  For one rank:
 *
 *   y[m] = sum over k of W[m][k] * x[k]      W: [M][K] bf16 row-major, x: [K]
 *
 * The definition is the exact real sum.  Computed here in binary64: every
 * product of two bfloat16 values (8-bit significands) is exact in binary64,
 * and the sequential sum over k adds at most K rounding errors of 2^-53
 * each, far below anything a binary32 kernel can resolve.
 */
void oracle_gemv_f64(const uint16_t *W, const uint16_t *x, size_t M, size_t K, double *y,
                     int threads)
{
    long long m;
#ifdef _OPENMP
    if (threads > 0)
        omp_set_num_threads(threads);
#pragma omp parallel for schedule(static) if (threads != 1)
#endif
    for (m = 0; m < (long long)M; ++m) {
        double s = 0.0;
        for (size_t k = 0; k < K; ++k)
            s += (double)widen_bf16(W[(size_t)m * K + k]) * (double)widen_bf16(x[k]);
        y[m] = s;
    }
    (void)threads;
}

/*
 * The op after the AllReduce in a decode layer ("vLLM 分布式推理核心" page,
 * sections 一 and 二: the compute stream resumes with the next LayerNorm once
 * the AllReduce completes).  The page names the op without defining it;
 * reading used here: the residual add followed by the RMS form of the layer
 * norm with a weight (no centring), as in the 70B-class decoders the page
 * targets:
 *
 *   h[i] = bf16_rne( f32(a[i]) + f32(res[i]) )          a = the AllReduce result
 *   y[i] = h[i] * gamma[i] / sqrt( (1/n) * sum_j h[j]^2 + eps )
 *
 * h is a plain binary32 addition rounded once, so it has one exact answer.
 * y is returned unrounded in binary64 (h, gamma exact; the sum of squares of
 * bf16 values is exact in binary64 up to n roundings of 2^-53); a kernel's
 * bf16 result is held to one bf16 ulp of it.
 */
void oracle_add_rmsnorm(const uint16_t *a, const uint16_t *res, const uint16_t *gamma, size_t n,
                        float eps, uint16_t *h_out, double *y_out)
{
    double ss = 0.0;
    for (size_t i = 0; i < n; ++i) {
        float s = widen_bf16(a[i]) + widen_bf16(res[i]);
        uint32_t bits;
        memcpy(&bits, &s, sizeof bits);
        h_out[i] = oracle_f32_to_bf16(bits);
        const double hv = (double)widen_bf16(h_out[i]);
        ss += hv * hv;
    }
    const double inv = 1.0 / sqrt(ss / (double)n + (double)eps);
    for (size_t i = 0; i < n; ++i)
        y_out[i] = (double)widen_bf16(h_out[i]) * (double)widen_bf16(gamma[i]) * inv;
}

/*
 * Reference for the atomic-lines variant ("微秒必争…" page, section
 * "四大核心机制", item 4: ranks add into shared blocks with hardware atomics,
 * so the order of the additions is the order of arrival).  No single
 * binary32 result is "the" answer; what such a sum fixes is its distance
 * from the exact sum: any order of N-1 binary32 additions of the N widened
 * values lies within gamma_{N-1} * sum_r |x_r| of it (recursive summation
 * bound, gamma_k = k u / (1 - k u), u = 2^-24).  This returns, per element,
 * the binary64 sum (left to right; for bf16 inputs it is the exact sum
 * unless the values span more than about 40 binades) and sum_r |x_r|.
 */
void oracle_sum_abs_f64(const uint16_t *const *in, int n_ranks, size_t n, double *sum,
                        double *abs_sum)
{
    for (size_t i = 0; i < n; ++i) {
        double s = 0.0, a = 0.0;
        for (int r = 0; r < n_ranks; ++r) {
            const double v = (double)widen_bf16(in[r][i]);
            s += v;
            a += fabs(v);
        }
        sum[i] = s;
        abs_sum[i] = a;
    }
}
