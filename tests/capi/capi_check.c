/*
 * Drives libddp.so through its C ABI alone (no Python, no torch): device
 * memory from hipMalloc, the default stream, and every entry point of
 * ddp.h on one seeded problem -- N = 4 ranks, 300 parameters of 1..5000
 * elements, a 64 KiB bucket cap -- checked bit for bit against the CPU
 * oracle's C core (test infrastructure, linked only here).
 *
 * Exit status 0 and "capi ok" on success; a message and status 1 otherwise.
 */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "ddp.h"

/* oracle core (tests only) */
int oracle_bucket_avg(const void *const *x, int N, int64_t len, int order, int in_dtype,
                      int out_dtype, void *out);
int oracle_sgd_step(float *p, float *m, const void *g, int g_dtype, int64_t n, float lr, float mu);
int oracle_accumulate(void *dst, const void *src, int dtype, int64_t n);

#define N 4
#define NP 300

#define CHECK_HIP(x)                                                              \
    do {                                                                          \
        hipError_t e_ = (x);                                                      \
        if (e_ != hipSuccess) {                                                   \
            fprintf(stderr, "%s:%d %s: %s\n", __FILE__, __LINE__, #x,             \
                    hipGetErrorString(e_));                                       \
            exit(1);                                                              \
        }                                                                         \
    } while (0)
#define CHECK_DDP(x)                                                              \
    do {                                                                          \
        ddp_status_t s_ = (x);                                                    \
        if (s_ != DDP_OK) {                                                       \
            fprintf(stderr, "%s:%d %s: %s (%s)\n", __FILE__, __LINE__, #x,        \
                    ddp_status_string(s_), ddp_last_error());                     \
            exit(1);                                                              \
        }                                                                         \
    } while (0)

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint32_t next_u32(void)
{   /* xorshift64*: seeded test data, not part of the method */
    rng_state ^= rng_state >> 12;
    rng_state ^= rng_state << 25;
    rng_state ^= rng_state >> 27;
    return (uint32_t)((rng_state * 0x2545F4914F6CDD1Dull) >> 32);
}
static float next_grad(void) { return ((float)(next_u32() >> 8) / 16777216.0f - 0.5f) * 2e-3f; }

static int same_bits(const void *a, const void *b, size_t n, const char *what)
{
    if (memcmp(a, b, n) != 0) {
        const uint32_t *x = a, *y = b;
        for (size_t i = 0; i < n / 4; ++i)
            if (x[i] != y[i]) {
                fprintf(stderr, "%s differs at word %zu: %08x vs %08x\n", what, i, x[i], y[i]);
                break;
            }
        return 0;
    }
    return 1;
}

int main(void)
{
    int64_t numel[NP];
    for (int p = 0; p < NP; ++p) numel[p] = 1 + (int64_t)(next_u32() % 5000);
    ddp_plan_t *plan = NULL;
    CHECK_DDP(ddp_plan_buckets(numel, NP, 64 << 10, DDP_F32, &plan));
    const int64_t P = ddp_plan_total(plan);
    const int32_t B = ddp_plan_num_buckets(plan);

    /* per-rank, per-parameter gradients on the host and device */
    float *hg[N][NP];
    void *dg[N][NP];
    for (int r = 0; r < N; ++r)
        for (int p = 0; p < NP; ++p) {
            hg[r][p] = malloc(sizeof(float) * numel[p]);
            for (int64_t j = 0; j < numel[p]; ++j) hg[r][p][j] = next_grad();
            CHECK_HIP(hipMalloc(&dg[r][p], sizeof(float) * numel[p]));
            CHECK_HIP(hipMemcpy(dg[r][p], hg[r][p], sizeof(float) * numel[p], hipMemcpyHostToDevice));
        }

    /* flatten every rank; the host-side flat layout from the plan queries */
    ddp_binding_t *bind[N];
    void *dflat[N];
    const void *cflat[N];
    float *hflat[N];
    for (int r = 0; r < N; ++r) {
        CHECK_DDP(ddp_bind_params(plan, dg[r], NULL, &bind[r]));
        CHECK_HIP(hipMalloc(&dflat[r], sizeof(float) * P));
        CHECK_DDP(ddp_flatten(plan, bind[r], -1, dflat[r], DDP_F32, NULL));
        cflat[r] = dflat[r];
        hflat[r] = malloc(sizeof(float) * P);
        for (int p = 0; p < NP; ++p) {
            int32_t b;
            int64_t off, base;
            CHECK_DDP(ddp_plan_param(plan, p, &b, &off));
            CHECK_DDP(ddp_plan_bucket(plan, b, NULL, &base, NULL, NULL));
            memcpy(hflat[r] + base + off, hg[r][p], sizeof(float) * numel[p]);
        }
    }
    float *got = malloc(sizeof(float) * P), *want = malloc(sizeof(float) * P);
    for (int r = 0; r < N; ++r) {
        CHECK_HIP(hipMemcpy(got, dflat[r], sizeof(float) * P, hipMemcpyDeviceToHost));
        if (!same_bits(got, hflat[r], sizeof(float) * P, "flatten")) return 1;
    }

    void *dout;
    CHECK_HIP(hipMalloc(&dout, sizeof(float) * P));
    CHECK_DDP(ddp_plan_prepare_ranks(plan, N));   /* the RING table for N ranks, up front */
    for (int order = DDP_ORDER_SEQUENTIAL; order <= DDP_ORDER_RING; ++order) {
        /* whole synchronisation in one launch */
        CHECK_DDP(ddp_sync_allreduce_avg(plan, cflat, N, (ddp_order_t)order, DDP_F32, dout, NULL));
        CHECK_HIP(hipDeviceSynchronize());
        CHECK_HIP(hipMemcpy(got, dout, sizeof(float) * P, hipMemcpyDeviceToHost));
        for (int32_t b = 0; b < B; ++b) {
            int64_t len, base;
            CHECK_DDP(ddp_plan_bucket(plan, b, &len, &base, NULL, NULL));
            const void *x[N];
            for (int r = 0; r < N; ++r) x[r] = hflat[r] + base;
            if (oracle_bucket_avg(x, N, len, order, 0, 0, want + base)) return 1;
        }
        if (!same_bits(got, want, sizeof(float) * P, "sync")) return 1;
        /* the same through per-bucket calls */
        for (int32_t b = 0; b < B; ++b) {
            int64_t len, base;
            CHECK_DDP(ddp_plan_bucket(plan, b, &len, &base, NULL, NULL));
            const void *x[N];
            for (int r = 0; r < N; ++r) x[r] = (const char *)dflat[r] + 4 * base;
            CHECK_DDP(ddp_bucket_allreduce_avg(x, N, len, (ddp_order_t)order, DDP_F32, DDP_F32,
                                               (char *)dout + 4 * base, NULL));
        }
        CHECK_HIP(hipMemcpy(got, dout, sizeof(float) * P, hipMemcpyDeviceToHost));
        if (!same_bits(got, want, sizeof(float) * P, "per-bucket")) return 1;
        /* the occupancy policy changes timing only */
        if (ddp_get_occupancy() != DDP_OCCUPANCY_TUNED) return 1;
        CHECK_DDP(ddp_set_occupancy(DDP_OCCUPANCY_SHARED));
        CHECK_DDP(ddp_sync_allreduce_avg(plan, cflat, N, (ddp_order_t)order, DDP_F32, dout, NULL));
        CHECK_DDP(ddp_set_occupancy(DDP_OCCUPANCY_TUNED));
        CHECK_HIP(hipMemcpy(got, dout, sizeof(float) * P, hipMemcpyDeviceToHost));
        if (!same_bits(got, want, sizeof(float) * P, "sync, shared occupancy")) return 1;
    }

    /* unflatten the ring average into fresh parameter buffers */
    void *dres[NP];
    for (int p = 0; p < NP; ++p) CHECK_HIP(hipMalloc(&dres[p], sizeof(float) * numel[p]));
    ddp_binding_t *rbind;
    CHECK_DDP(ddp_bind_params(plan, dres, NULL, &rbind));
    CHECK_DDP(ddp_unflatten(plan, rbind, -1, dout, DDP_F32, NULL));
    CHECK_HIP(hipDeviceSynchronize());
    for (int p = 0; p < NP; ++p) {
        int32_t b;
        int64_t off, base;
        CHECK_DDP(ddp_plan_param(plan, p, &b, &off));
        CHECK_DDP(ddp_plan_bucket(plan, b, NULL, &base, NULL, NULL));
        CHECK_HIP(hipMemcpy(got, dres[p], sizeof(float) * numel[p], hipMemcpyDeviceToHost));
        if (!same_bits(got, want + base + off, sizeof(float) * numel[p], "unflatten")) return 1;
    }

    /* the same step in one kernel over the per-parameter gradients */
    ddp_param_sync_t *ps;
    CHECK_DDP(ddp_param_sync_create(plan, (const ddp_binding_t *const *)bind, N, rbind,
                                    DDP_ORDER_RING, DDP_F32, &ps));
    for (int p = 0; p < NP; ++p) CHECK_HIP(hipMemset(dres[p], 0xff, sizeof(float) * numel[p]));
    CHECK_DDP(ddp_param_sync_run(ps, NULL));
    CHECK_HIP(hipDeviceSynchronize());
    for (int p = 0; p < NP; ++p) {
        int32_t b;
        int64_t off, base;
        CHECK_DDP(ddp_plan_param(plan, p, &b, &off));
        CHECK_DDP(ddp_plan_bucket(plan, b, NULL, &base, NULL, NULL));
        CHECK_HIP(hipMemcpy(got, dres[p], sizeof(float) * numel[p], hipMemcpyDeviceToHost));
        if (!same_bits(got, want + base + off, sizeof(float) * numel[p], "param sync")) return 1;
    }
    ddp_param_sync_free(ps);

    /* fused momentum-SGD step on flat parameters */
    float *hp = malloc(sizeof(float) * P), *hm = calloc((size_t)P, sizeof(float));
    for (int64_t i = 0; i < P; ++i) hp[i] = next_grad() * 1000.0f;
    void *dp, *dm;
    CHECK_HIP(hipMalloc(&dp, sizeof(float) * P));
    CHECK_HIP(hipMalloc(&dm, sizeof(float) * P));
    CHECK_HIP(hipMemcpy(dp, hp, sizeof(float) * P, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemset(dm, 0, sizeof(float) * P));
    CHECK_DDP(ddp_sync_sgd_update(plan, cflat, N, DDP_ORDER_RING, DDP_F32, NULL, dp, dm, 0.1f, 0.9f,
                                  NULL));
    CHECK_HIP(hipDeviceSynchronize());
    oracle_sgd_step(hp, hm, want, 0, P, 0.1f, 0.9f);   /* want holds the ring average */
    CHECK_HIP(hipMemcpy(got, dp, sizeof(float) * P, hipMemcpyDeviceToHost));
    if (!same_bits(got, hp, sizeof(float) * P, "sgd params")) return 1;
    CHECK_HIP(hipMemcpy(got, dm, sizeof(float) * P, hipMemcpyDeviceToHost));
    if (!same_bits(got, hm, sizeof(float) * P, "sgd momentum")) return 1;

    /* the same step on per-parameter parameters and momentum buffers */
    void *dpp[NP], *dpm[NP];
    float *hpp = malloc(sizeof(float) * P), *hpm = calloc((size_t)P, sizeof(float));
    for (int p = 0; p < NP; ++p) {
        int32_t b;
        int64_t off, base;
        CHECK_DDP(ddp_plan_param(plan, p, &b, &off));
        CHECK_DDP(ddp_plan_bucket(plan, b, NULL, &base, NULL, NULL));
        for (int64_t j = 0; j < numel[p]; ++j) hpp[base + off + j] = next_grad() * 1000.0f;
        CHECK_HIP(hipMalloc(&dpp[p], sizeof(float) * numel[p]));
        CHECK_HIP(hipMalloc(&dpm[p], sizeof(float) * numel[p]));
        CHECK_HIP(hipMemcpy(dpp[p], hpp + base + off, sizeof(float) * numel[p],
                            hipMemcpyHostToDevice));
        CHECK_HIP(hipMemset(dpm[p], 0, sizeof(float) * numel[p]));
    }
    ddp_binding_t *pbind, *mbind;
    CHECK_DDP(ddp_bind_params(plan, dpp, NULL, &pbind));
    CHECK_DDP(ddp_bind_params(plan, dpm, NULL, &mbind));
    ddp_param_sync_t *psgd;
    CHECK_DDP(ddp_param_sgd_create(plan, (const ddp_binding_t *const *)bind, N, NULL, pbind, mbind,
                                   DDP_ORDER_RING, DDP_F32, &psgd));
    CHECK_DDP(ddp_param_sgd_run(psgd, 0.1f, 0.9f, NULL));
    CHECK_HIP(hipDeviceSynchronize());
    oracle_sgd_step(hpp, hpm, want, 0, P, 0.1f, 0.9f);   /* flat order: want is the flat average */
    for (int p = 0; p < NP; ++p) {
        int32_t b;
        int64_t off, base;
        CHECK_DDP(ddp_plan_param(plan, p, &b, &off));
        CHECK_DDP(ddp_plan_bucket(plan, b, NULL, &base, NULL, NULL));
        CHECK_HIP(hipMemcpy(got, dpp[p], sizeof(float) * numel[p], hipMemcpyDeviceToHost));
        if (!same_bits(got, hpp + base + off, sizeof(float) * numel[p], "param sgd params")) return 1;
        CHECK_HIP(hipMemcpy(got, dpm[p], sizeof(float) * numel[p], hipMemcpyDeviceToHost));
        if (!same_bits(got, hpm + base + off, sizeof(float) * numel[p], "param sgd momentum")) return 1;
    }
    if (ddp_param_sync_run(psgd, NULL) != DDP_ERR_INVALID_ARG) return 1;   /* wrong kind */
    ddp_param_sync_free(psgd);
    ddp_binding_free(pbind);
    ddp_binding_free(mbind);

    /* accumulate rank 1 into rank 0 and rank 3 into rank 2 */
    void *adst[2] = {dflat[0], dflat[2]};
    const void *asrc[2] = {dflat[1], dflat[3]};
    CHECK_DDP(ddp_accumulate(adst, asrc, 2, P, DDP_F32, NULL));
    CHECK_HIP(hipDeviceSynchronize());
    oracle_accumulate(hflat[0], hflat[1], 0, P);
    oracle_accumulate(hflat[2], hflat[3], 0, P);
    CHECK_HIP(hipMemcpy(got, dflat[0], sizeof(float) * P, hipMemcpyDeviceToHost));
    if (!same_bits(got, hflat[0], sizeof(float) * P, "accumulate 0")) return 1;
    CHECK_HIP(hipMemcpy(got, dflat[2], sizeof(float) * P, hipMemcpyDeviceToHost));
    if (!same_bits(got, hflat[2], sizeof(float) * P, "accumulate 2")) return 1;

    /* errors come back as status codes */
    if (ddp_sync_allreduce_avg(plan, cflat, 0, DDP_ORDER_RING, DDP_F32, dout, NULL) !=
        DDP_ERR_INVALID_ARG)
        return 1;
    if (ddp_plan_prepare_ranks(plan, DDP_MAX_RANKS + 1) != DDP_ERR_INVALID_ARG) return 1;
    if (ddp_set_occupancy((ddp_occupancy_t)7) != DDP_ERR_INVALID_ARG) return 1;

    ddp_binding_free(rbind);
    for (int r = 0; r < N; ++r) ddp_binding_free(bind[r]);
    ddp_plan_free(plan);
    printf("capi ok: N=%d, %d parameters, %lld elements, %d buckets\n", N, NP, (long long)P, B);
    return 0;
}
