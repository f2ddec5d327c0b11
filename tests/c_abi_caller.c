/*
 * A plain C caller of the C ABI (include/ar.h), built with a C compiler
 * against the HIP runtime API only -- no Python, no torch.  It initialises 4
 * ranks, runs a one-shot LL and a two-shot DIRECT AllReduce of small
 * integers (their sums are exact in binary32 and in bf16, so the expected
 * output is the integer sum written as bf16), checks every rank's copy,
 * exercises the error codes and the step end, and tears down.
 * Exit status 0 and "c caller ok" on success.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "ar.h"

#define N_RANKS 4
#define N_ELEMS 4104          /* a multiple of 8 that ends in a ragged tile */

static int fails = 0;

#define EXPECT(cond, what)                                                   \
    do {                                                                     \
        if (!(cond)) {                                                       \
            fprintf(stderr, "c caller: %s failed (line %d)\n", what, __LINE__); \
            ++fails;                                                         \
        }                                                                    \
    } while (0)

#define HIP_OK(call)                                                         \
    do {                                                                     \
        hipError_t e_ = (call);                                              \
        if (e_ != hipSuccess) {                                              \
            fprintf(stderr, "c caller: %s -> HIP error %d\n", #call, (int)e_); \
            return 2;                                                        \
        }                                                                    \
    } while (0)

/* integer v with |v| < 256 as a bf16 pattern: exact (8 significant bits) */
static uint16_t bf16_of_int(int v)
{
    float f = (float)v;
    uint32_t b;
    memcpy(&b, &f, sizeof b);
    return (uint16_t)(b >> 16);
}

static int value(int rank, int i) { return (i * 7 + rank * 13) % 31 - 15; }

static int run(int algo, int proto, uint32_t epoch, void *const *ins, void *out, uint16_t *host)
{
    if (ar_set_options(algo, proto) != AR_OK)
        return -1;
    int rc = ar_allreduce((const void *const *)ins, out, N_ELEMS, epoch, 0);
    if (rc != AR_OK)
        return rc;
    if (hipDeviceSynchronize() != hipSuccess)
        return -2;
    if (hipMemcpy(host, out, sizeof(uint16_t) * N_RANKS * N_ELEMS, hipMemcpyDeviceToHost) !=
        hipSuccess)
        return -3;
    int bad = 0;
    for (int r = 0; r < N_RANKS; ++r)
        for (int i = 0; i < N_ELEMS; ++i) {
            int sum = 0;
            for (int s = 0; s < N_RANKS; ++s)
                sum += value(s, i);
            if (host[(size_t)r * N_ELEMS + i] != bf16_of_int(sum))
                ++bad;
        }
    return bad;
}

int main(void)
{
    static uint16_t host[N_RANKS * N_ELEMS];
    void *ins[N_RANKS];
    void *out = NULL;

    EXPECT(ar_init(0, 16) == AR_ERR_INVALID, "ar_init(0 ranks)");
    EXPECT(ar_destroy() == AR_ERR_NOT_INIT, "ar_destroy before init");
    if (ar_init(N_RANKS, N_ELEMS) != AR_OK) {
        fprintf(stderr, "c caller: ar_init failed: %s\n", ar_strerror(AR_ERR_HIP));
        return 2;
    }
    EXPECT(ar_init(N_RANKS, N_ELEMS) == AR_ERR_STATE, "second ar_init");
    for (int r = 0; r < N_RANKS; ++r) {
        for (int i = 0; i < N_ELEMS; ++i)
            host[i] = bf16_of_int(value(r, i));
        HIP_OK(hipMalloc(&ins[r], sizeof(uint16_t) * N_ELEMS));
        HIP_OK(hipMemcpy(ins[r], host, sizeof(uint16_t) * N_ELEMS, hipMemcpyHostToDevice));
    }
    HIP_OK(hipMalloc(&out, sizeof(uint16_t) * N_RANKS * N_ELEMS));

    EXPECT(run(AR_ALGO_ONESHOT, AR_PROTO_LL, 1, ins, out, host) == 0, "one-shot LL sums");
    EXPECT(run(AR_ALGO_TWOSHOT, AR_PROTO_DIRECT, 2, ins, out, host) == 0, "two-shot DIRECT sums");
    /* the epoch sequence and the argument checks */
    EXPECT(ar_allreduce((const void *const *)ins, out, N_ELEMS, 7, 0) == AR_ERR_INVALID,
           "epoch out of sequence");
    EXPECT(ar_allreduce((const void *const *)ins, out, 12, 3, 0) == AR_ERR_INVALID, "n % 8");
    EXPECT(ar_set_options(AR_ALGO_TWOSHOT, AR_PROTO_LL) == AR_ERR_INVALID, "two-shot LL");
    EXPECT(ar_step_end(0) == AR_OK, "ar_step_end after 2 calls");
    EXPECT(run(AR_ALGO_AUTO, AR_PROTO_AUTO, 1, ins, out, host) == 0, "AUTO after the step end");
    uint32_t st[4] = {1, 1, 1, 1};
    EXPECT(ar_get_status(st) == AR_OK && st[0] == 0, "status clean");
    EXPECT(ar_query(0, 0) == N_RANKS, "query ranks");
    EXPECT(ar_strerror(AR_ERR_TIMEOUT) != NULL && ar_strerror(AR_ERR_TIMEOUT)[0] != 0, "strerror");

    for (int r = 0; r < N_RANKS; ++r)
        HIP_OK(hipFree(ins[r]));
    HIP_OK(hipFree(out));
    EXPECT(ar_destroy() == AR_OK, "ar_destroy");
    EXPECT(ar_destroy() == AR_ERR_NOT_INIT, "second ar_destroy");
    if (fails) {
        fprintf(stderr, "c caller: %d checks failed\n", fails);
        return 1;
    }
    printf("c caller ok\n");
    return 0;
}
