/*
 * capi_demo.c -- the library driven from plain C99 through include/zsp.h
 * alone: no Python, no torch. Device memory comes from the HIP runtime's C
 * API. A small padded parameter list at N_d = 5 goes through partition, copy-in,
 * three fused reduce + Adam + cast steps over every virtual rank, a gather
 * of every parameter into one buffer and list gathers into separate
 * outputs; each result is compared bit for bit with the
 * CPU oracle (test infrastructure, linked only into this test program).
 * A few argument errors are checked too. Prints "capi demo ok ..." and
 * exits 0, or names the first difference and exits 1. With --host-only it
 * stops after the checks that need no GPU (argument errors, layout queries).
 *
 * Inputs come from SplitMix64 (Steele, Lea and Flood, "Fast splittable
 * pseudorandom number generators", 2014) on a counter; gradients carry a
 * NaN in every pad slot of the full padded layout, which must never be read.
 */
#define __HIP_PLATFORM_AMD__ 1
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "oracle.h"
#include "zsp.h"

#define ND 5
#define T 6
#define STEPS 3
#define LIST_N (T + 70)

static const int64_t NUMEL[T] = {1003, 64, 5, 0, 3 * 4096 + 1, 4096 * 4 + 7};

static uint64_t splitmix64(uint64_t x) {
    x += 0x9E3779B97F4A7C15ull;
    x = (x ^ (x >> 30)) * 0xBF58476D1CE4E5B9ull;
    x = (x ^ (x >> 27)) * 0x94D049BB133111EBull;
    return x ^ (x >> 31);
}

/* A bf16 value in (-scale, scale): a uniform draw, truncated to bf16. */
static uint16_t draw_bf16(uint64_t stream, uint64_t i, float scale) {
    const uint64_t r = splitmix64((stream << 40) ^ i);
    const float u = (float)((double)(r >> 11) * (1.0 / 9007199254740992.0));  /* [0, 1) */
    const float x = (2.0f * u - 1.0f) * scale;
    uint32_t bits;
    memcpy(&bits, &x, 4);
    return (uint16_t)(bits >> 16);
}

static int fail_hip(hipError_t e, const char* what) {
    printf("HIP error %d (%s) in %s\n", (int)e, hipGetErrorString(e), what);
    return 1;
}

#define HIPCK(call) do { hipError_t e_ = (call); if (e_ != hipSuccess) return fail_hip(e_, #call); } while (0)
#define ZCK(call) do { zsp_status s_ = (call); if (s_ != ZSP_OK) { \
    printf("%s -> %d: %s\n", #call, (int)s_, zsp_last_error()); return 1; } } while (0)

static int same(const void* a, const void* b, size_t n, const char* what) {
    if (memcmp(a, b, n) == 0) return 0;
    const unsigned char* x = (const unsigned char*)a;
    const unsigned char* y = (const unsigned char*)b;
    size_t i = 0;
    while (x[i] == y[i]) ++i;
    printf("%s differs from the oracle at byte %zu\n", what, i);
    return 1;
}

static int run(int host_only) {
    /* argument errors: checked on the host, nothing enqueued */
    zsp_plan* bad = NULL;
    if (zsp_partition(NUMEL, T, 0, &bad) != ZSP_EINVAL || bad != NULL || !zsp_last_error()[0]) {
        printf("n_d = 0 was not refused\n");
        return 1;
    }
    zsp_plan* P = NULL;
    ZCK(zsp_partition(NUMEL, T, ND, &P));
    if (zsp_gather(P, T, ZSP_SRC_WORK, NULL, NULL) != ZSP_ERANGE) {
        printf("a parameter id past the end was not refused\n");
        return 1;
    }
    if (zsp_adam_step(P, ZSP_ALL_RANKS, 1e-3f, 0.9f, 0.999f, 1e-8f, 1, NULL) != ZSP_ESTATE) {
        printf("a step on an unbound plan was not refused\n");
        return 1;
    }

    int64_t S = 0, padded = 0, numel = 0, state_bytes = 0;
    ZCK(zsp_plan_info(P, &S, &padded, &state_bytes));
    for (int t = 0; t < T; ++t) numel += NUMEL[t];
    int64_t o_pad[T], o_sl[T], o_full[T + 1], o_shard[T + 1], o_flat[T + 1], o_S = 0;
    if (orc_layout(T, NUMEL, ND, o_pad, o_sl, o_full, o_shard, o_flat, &o_S) != 0) return 1;
    if (S != o_S || padded != o_full[T] || numel != o_flat[T] || state_bytes != 16 * S) {
        printf("plan sizes differ from the oracle's layout\n");
        return 1;
    }
    for (int t = 0; t < T; ++t) {
        int64_t n, pad, sl, fo, so;
        ZCK(zsp_plan_tensor(P, t, &n, &pad, &sl, &fo, &so));
        if (n != NUMEL[t] || pad != o_pad[t] || sl != o_sl[t] || fo != o_full[t] ||
            so != o_shard[t]) {
            printf("parameter %d: layout differs from the oracle's\n", t);
            return 1;
        }
    }
    if (host_only) {
        zsp_destroy(P);
        printf("capi demo host checks ok: %d parameters, N_d = %d, S = %lld\n", T, ND,
               (long long)S);
        return 0;
    }

    const int64_t n_state = (int64_t)ND * S;
    float* h_master = malloc(sizeof(float) * n_state);
    float* h_m = malloc(sizeof(float) * n_state);
    float* h_v = malloc(sizeof(float) * n_state);
    uint16_t* h_work = malloc(sizeof(uint16_t) * n_state);
    float* o_master = malloc(sizeof(float) * n_state);
    float* o_m = malloc(sizeof(float) * n_state);
    float* o_v = malloc(sizeof(float) * n_state);
    uint16_t* o_work = malloc(sizeof(uint16_t) * n_state);
    float* o_red = malloc(sizeof(float) * (S > 0 ? S : 1));
    uint16_t* params = malloc(sizeof(uint16_t) * numel);
    uint16_t* gathered = malloc(sizeof(uint16_t) * numel);
    uint16_t* o_gathered = malloc(sizeof(uint16_t) * numel);
    uint16_t* grads[ND];
    for (int r = 0; r < ND; ++r) grads[r] = malloc(sizeof(uint16_t) * padded);

    for (int64_t i = 0; i < numel; ++i) params[i] = draw_bf16(1, (uint64_t)i, 0.05f);

    float *d_master, *d_m, *d_v;
    uint16_t *d_work, *d_params, *d_out;
    void* d_grads[ND];
    HIPCK(hipMalloc((void**)&d_master, sizeof(float) * n_state));
    HIPCK(hipMalloc((void**)&d_m, sizeof(float) * n_state));
    HIPCK(hipMalloc((void**)&d_v, sizeof(float) * n_state));
    HIPCK(hipMalloc((void**)&d_work, sizeof(uint16_t) * n_state));
    HIPCK(hipMalloc((void**)&d_params, sizeof(uint16_t) * numel));
    HIPCK(hipMalloc((void**)&d_out, sizeof(uint16_t) * numel));
    for (int r = 0; r < ND; ++r) HIPCK(hipMalloc(&d_grads[r], sizeof(uint16_t) * padded));
    HIPCK(hipMemcpy(d_params, params, sizeof(uint16_t) * numel, hipMemcpyHostToDevice));

    ZCK(zsp_bind_state(P, ZSP_ALL_RANKS, d_master, d_m, d_v, d_work, NULL));
    ZCK(zsp_load_params(P, d_params, ZSP_BF16, NULL));
    if (orc_partition(T, NUMEL, ND, 0, ND, params, ORC_BF16, o_master, o_work, o_m, o_v) != 0)
        return 1;

    const float lr = 1e-3f, b1 = 0.9f, b2 = 0.999f, eps = 1e-8f;
    for (int step = 1; step <= STEPS; ++step) {
        for (int r = 0; r < ND; ++r) {
            for (int64_t i = 0; i < padded; ++i) grads[r][i] = 0x7FC0; /* NaN: pads */
            for (int t = 0; t < T; ++t)
                for (int64_t k = 0; k < NUMEL[t]; ++k)
                    grads[r][o_full[t] + k] =
                        draw_bf16(100 + 10 * (uint64_t)step + (uint64_t)r,
                                  (uint64_t)(o_full[t] + k), 0.01f);
            HIPCK(hipMemcpy(d_grads[r], grads[r], sizeof(uint16_t) * padded,
                            hipMemcpyHostToDevice));
        }
        ZCK(zsp_reduce_adam_step(P, ZSP_ALL_RANKS, (const void* const*)d_grads, ZSP_BF16,
                                 ZSP_GRADS_FULL, 0, lr, b1, b2, eps, step, NULL));
        for (int j = 0; j < ND; ++j) {
            const int64_t at = (int64_t)j * S;
            if (orc_reduce(T, NUMEL, ND, j, (const void* const*)grads, ORC_BF16, ORC_GRADS_FULL,
                           o_red) != 0 ||
                orc_adam(T, NUMEL, ND, j, o_master + at, o_m + at, o_v + at, o_work + at, o_red,
                         lr, b1, b2, eps, step) != 0)
                return 1;
        }
    }
    ZCK(zsp_gather_range(P, 0, T, ZSP_SRC_WORK, d_out, NULL));
    /* The list form: every parameter in reverse order (kernel-argument
     * form), then 70 entries cycling through them (staged form), each into
     * an output of its own; empty parameters take NULL. */
    int32_t ids[LIST_N];
    void* d_lists[LIST_N];
    for (int i = 0; i < LIST_N; ++i) {
        ids[i] = i < T ? T - 1 - i : (int32_t)((7 * i) % T);
        d_lists[i] = NULL;
        if (NUMEL[ids[i]] > 0)
            HIPCK(hipMalloc(&d_lists[i], sizeof(uint16_t) * (size_t)NUMEL[ids[i]]));
    }
    ZCK(zsp_gather_many(P, ids, T, ZSP_SRC_WORK, d_lists, NULL));
    ZCK(zsp_gather_many(P, ids + T, LIST_N - T, ZSP_SRC_WORK, d_lists + T, NULL));
    HIPCK(hipDeviceSynchronize());
    HIPCK(hipMemcpy(h_master, d_master, sizeof(float) * n_state, hipMemcpyDeviceToHost));
    HIPCK(hipMemcpy(h_m, d_m, sizeof(float) * n_state, hipMemcpyDeviceToHost));
    HIPCK(hipMemcpy(h_v, d_v, sizeof(float) * n_state, hipMemcpyDeviceToHost));
    HIPCK(hipMemcpy(h_work, d_work, sizeof(uint16_t) * n_state, hipMemcpyDeviceToHost));
    HIPCK(hipMemcpy(gathered, d_out, sizeof(uint16_t) * numel, hipMemcpyDeviceToHost));
    for (int t = 0; t < T; ++t)
        if (orc_gather(T, NUMEL, ND, t, o_work, ORC_BF16, o_gathered + o_flat[t]) != 0) return 1;

    int bad_count = same(h_master, o_master, sizeof(float) * n_state, "master") +
                    same(h_m, o_m, sizeof(float) * n_state, "m") +
                    same(h_v, o_v, sizeof(float) * n_state, "v") +
                    same(h_work, o_work, sizeof(uint16_t) * n_state, "work") +
                    same(gathered, o_gathered, sizeof(uint16_t) * numel, "gather");
    for (int i = 0; i < LIST_N; ++i) {
        const int t = ids[i];
        if (!d_lists[i]) continue;
        HIPCK(hipMemcpy(gathered, d_lists[i], sizeof(uint16_t) * (size_t)NUMEL[t],
                        hipMemcpyDeviceToHost));
        bad_count += same(gathered, o_gathered + o_flat[t], sizeof(uint16_t) * (size_t)NUMEL[t],
                          i < T ? "list gather (arguments)" : "list gather (staged)");
    }
    /* The staged list again, prepared once (records built on the device)
     * and run twice into outputs wiped before each run. */
    zsp_gather_list* G = NULL;
    ZCK(zsp_gather_list_create(P, ids + T, LIST_N - T, ZSP_SRC_WORK, d_lists + T, NULL, &G));
    for (int run = 0; run < 2; ++run) {
        for (int i = T; i < LIST_N; ++i)
            if (d_lists[i]) HIPCK(hipMemset(d_lists[i], 0xff, sizeof(uint16_t) * (size_t)NUMEL[ids[i]]));
        ZCK(zsp_gather_list_run(G, NULL));
        HIPCK(hipDeviceSynchronize());
        for (int i = T; i < LIST_N; ++i) {
            const int t = ids[i];
            if (!d_lists[i]) continue;
            HIPCK(hipMemcpy(gathered, d_lists[i], sizeof(uint16_t) * (size_t)NUMEL[t],
                            hipMemcpyDeviceToHost));
            bad_count += same(gathered, o_gathered + o_flat[t],
                              sizeof(uint16_t) * (size_t)NUMEL[t], "prepared list gather");
        }
    }
    zsp_gather_list_destroy(G);
    for (int i = 0; i < LIST_N; ++i) hipFree(d_lists[i]);
    zsp_destroy(P);
    hipFree(d_master);
    hipFree(d_m);
    hipFree(d_v);
    hipFree(d_work);
    hipFree(d_params);
    hipFree(d_out);
    for (int r = 0; r < ND; ++r) {
        hipFree(d_grads[r]);
        free(grads[r]);
    }
    free(h_master); free(h_m); free(h_v); free(h_work);
    free(o_master); free(o_m); free(o_v); free(o_work); free(o_red);
    free(params); free(gathered); free(o_gathered);
    if (bad_count) return 1;
    printf("capi demo ok: %d parameters, N_d = %d, S = %lld, %d fused steps + range, "
           "list and prepared list gathers, bit-exact\n", T, ND, (long long)S, STEPS);
    return 0;
}

/* --host-only: the argument and layout checks, which need no GPU. */
int main(int argc, char** argv) {
    return run(argc > 1 && strcmp(argv[1], "--host-only") == 0);
}
