/*
 * oracle.c -- plain CPU oracle for the per-rank hot path of ZeRO-3
 * intra-layer partitioning. TEST INFRASTRUCTURE ONLY (see oracle.h): the
 * product path never includes, links or calls this file.
 *
 * Written to be read against the pages, not to be fast: one element at a
 * time, no blocking, no vectorisation, no threads.
 *
 * Floating point: every operation is one fp32 IEEE-754 operation rounded to
 * nearest-even, in the order written. Build with -ffp-contract=off and
 * without fast-math; on x86-64 float arithmetic is SSE, so there is no excess
 * precision. Division and square root are the correctly rounded IEEE ones.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------ */
/* Scalar helpers                                                      */
/* ------------------------------------------------------------------ */

static float f32_from_bits(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t bits_from_f32(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

/* bf16 is the top half of an fp32 pattern, so widening is exact. */
static float bf16_to_f32(uint16_t h) { return f32_from_bits((uint32_t)h << 16); }

/* Narrowing fp32 -> bf16 keeps the top 16 bits and rounds on the 16 bits that
 * are dropped: round up when they exceed half an ulp of the result, or equal
 * half and the kept part is odd (ties to even). A carry out of the mantissa
 * moves to the next binade and past the largest finite value gives infinity,
 * as IEEE rounding requires. NaN stays NaN (quiet bit set). */
uint16_t orc_bf16_rne(float x) {
    uint32_t u = bits_from_f32(x);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t kept = u >> 16;
    uint32_t dropped = u & 0xffffu;
    if (dropped > 0x8000u || (dropped == 0x8000u && (kept & 1u))) kept += 1u;
    return (uint16_t)kept;
}

void orc_bf16_rne_array(int64_t n, const float* x, uint16_t* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = orc_bf16_rne(x[i]);
}

static float load_as_f32(const void* base, int64_t idx, int32_t dtype) {
    if (dtype == ORC_BF16) return bf16_to_f32(((const uint16_t*)base)[idx]);
    return ((const float*)base)[idx];
}

/* ------------------------------------------------------------------ */
/* Layout ([ZD] section 2; [ZST] "What stage 1 partitions")            */
/* ------------------------------------------------------------------ */

/* [ZD] section 2: padding makes a flattened parameter's length a multiple of
 * the rank count; the pad is the smallest number of elements that does so,
 * zero when the length already is a multiple. */
int64_t orc_pad(int64_t numel, int32_t nd) {
    int64_t rem = numel % nd;
    return rem == 0 ? 0 : (int64_t)nd - rem;
}

/* Every tensor is flattened and padded on its own; rank r owns the
 * contiguous slice [r*s, (r+1)*s) of each padded tensor, s = padded/nd
 * ([ZST] "What stage 1 partitions": rank i owns [i*N/P, (i+1)*N/P)).
 * A rank stores its slices one after another in tensor order (shard_off);
 * a full-layout buffer stores whole padded tensors one after another
 * (full_off); the unpadded concatenation uses flat_off. */
int orc_layout(int32_t T, const int64_t* numel, int32_t nd,
               int64_t* pad, int64_t* shard_len,
               int64_t* full_off, int64_t* shard_off, int64_t* flat_off,
               int64_t* S) {
    if (T < 0 || nd < 1 || (T > 0 && !numel)) return -1;
    full_off[0] = 0;
    shard_off[0] = 0;
    flat_off[0] = 0;
    for (int32_t t = 0; t < T; ++t) {
        if (numel[t] < 0) return -1;
        int64_t p = orc_pad(numel[t], nd);
        int64_t padded = numel[t] + p;
        pad[t] = p;
        shard_len[t] = padded / nd;
        full_off[t + 1] = full_off[t] + padded;
        shard_off[t + 1] = shard_off[t] + shard_len[t];
        flat_off[t + 1] = flat_off[t] + numel[t];
    }
    *S = shard_off[T];
    return 0;
}

/* [ZS3] equation M_Stage3: 16 bytes of model state per parameter, split as
 * 16-bit working parameter (2) + 16-bit gradient (2) + fp32 master (4) +
 * fp32 first and second Adam moments (4 + 4); a rank holds 1/N_d of it. */
int64_t orc_model_state_bytes(int64_t shard_elems) {
    return shard_elems * (2 + 2 + 4 + 4 + 4);
}

int64_t orc_stage_state_bytes(int32_t stage, int64_t psi, int64_t shard_elems,
                              int32_t grad_bytes) {
    const int64_t param_b = 2, optim_b = 4 + 4 + 4;  /* master, m, v */
    /* count of parameters each term is held for: all of them when
     * replicated, the rank's own slice when sharded */
    const int64_t params_n = stage >= 3 ? shard_elems : psi;
    const int64_t grads_n = stage >= 2 ? shard_elems : psi;
    const int64_t optim_n = stage >= 1 ? shard_elems : psi;
    if (stage < 0 || stage > 3) return -1;
    return param_b * params_n + (int64_t)grad_bytes * grads_n + optim_b * optim_n;
}

double orc_stage_comm_elems(int32_t stage, int64_t n, int32_t p) {
    if (p < 1 || n < 0) return -1.0;
    const double reduce_scatter = (double)n * (double)(p - 1) / (double)p;
    const double all_gather = reduce_scatter;
    const double all_reduce = reduce_scatter + all_gather;
    switch (stage) {
        case 0: return all_reduce;
        case 1: return all_reduce + all_gather;
        case 2: return reduce_scatter + all_gather;
        case 3: return reduce_scatter + 2.0 * all_gather;
        default: return -1.0;
    }
}

typedef struct {
    int64_t *pad, *shard_len, *full_off, *shard_off, *flat_off;
    int64_t S;
    void* block;
} layout_t;

static int layout_make(int32_t T, const int64_t* numel, int32_t nd, layout_t* L) {
    size_t n = (size_t)(T > 0 ? T : 0);
    int64_t* b = (int64_t*)malloc(sizeof(int64_t) * (5 * n + 3));
    if (!b) return -1;
    L->block = b;
    L->pad = b;
    L->shard_len = b + n;
    L->full_off = b + 2 * n;
    L->shard_off = b + 3 * n + 1;
    L->flat_off = b + 4 * n + 2;
    if (orc_layout(T, numel, nd, L->pad, L->shard_len, L->full_off, L->shard_off,
                   L->flat_off, &L->S) != 0) {
        free(b);
        return -1;
    }
    return 0;
}

static void layout_free(layout_t* L) { free(L->block); }

/* ------------------------------------------------------------------ */
/* Copy-in ([ZD] section 2, steps 1-4)                                 */
/* ------------------------------------------------------------------ */

/* Rank r's element i of tensor t is element k = r*s_t + i of the padded
 * flattened tensor; k >= numel_t is pad and holds zero. The fp32 master is
 * the parameter widened to fp32; the bf16 working copy is the parameter
 * itself (bf16 input) or its round-to-nearest-even narrowing (fp32 input);
 * the Adam moments start at zero. */
int orc_partition(int32_t T, const int64_t* numel, int32_t nd,
                  int32_t rank_lo, int32_t rank_hi,
                  const void* flat, int32_t dtype,
                  float* master, uint16_t* work, float* m, float* v) {
    if (rank_lo < 0 || rank_hi > nd || rank_lo > rank_hi) return -1;
    if (dtype != ORC_F32 && dtype != ORC_BF16) return -1;
    layout_t L;
    if (layout_make(T, numel, nd, &L) != 0) return -1;
    for (int32_t r = rank_lo; r < rank_hi; ++r) {
        int64_t base = (int64_t)(r - rank_lo) * L.S;
        for (int32_t t = 0; t < T; ++t) {
            int64_t s = L.shard_len[t];
            for (int64_t i = 0; i < s; ++i) {
                int64_t k = (int64_t)r * s + i;
                int64_t e = base + L.shard_off[t] + i;
                if (k < numel[t]) {
                    int64_t src = L.flat_off[t] + k;
                    float x = load_as_f32(flat, src, dtype);
                    master[e] = x;
                    work[e] = (dtype == ORC_BF16) ? ((const uint16_t*)flat)[src]
                                                  : orc_bf16_rne(x);
                } else {
                    master[e] = 0.0f;
                    work[e] = 0;
                }
                m[e] = 0.0f;
                v[e] = 0.0f;
            }
        }
    }
    layout_free(&L);
    return 0;
}

/* ------------------------------------------------------------------ */
/* Reduce ([ZD] section 3; [ZST] "Stage 2 also partitions gradients")  */
/* ------------------------------------------------------------------ */

/* Reduce-scatter sums the ranks' gradients and leaves each rank the summed
 * slice it owns. The sum starts from rank 0's value and adds ranks 1..nd-1
 * in order, one fp32 rounding per addition. */
static float sum_ranks(const float* g, int32_t nd) {
    float acc = g[0];
    for (int32_t r = 1; r < nd; ++r) acc = acc + g[r];
    return acc;
}

int orc_reduce(int32_t T, const int64_t* numel, int32_t nd, int32_t j,
               const void* const* grads, int32_t dtype, int32_t layout,
               float* out) {
    if (j < 0 || j >= nd) return -1;
    if (dtype != ORC_F32 && dtype != ORC_BF16) return -1;
    if (layout != ORC_GRADS_FULL && layout != ORC_GRADS_SHARD) return -1;
    layout_t L;
    if (layout_make(T, numel, nd, &L) != 0) return -1;
    float* vals = (float*)malloc(sizeof(float) * (size_t)nd);
    if (!vals) { layout_free(&L); return -1; }
    for (int32_t t = 0; t < T; ++t) {
        int64_t s = L.shard_len[t];
        for (int64_t i = 0; i < s; ++i) {
            int64_t k = (int64_t)j * s + i;          /* index in padded tensor t */
            int64_t e = L.shard_off[t] + i;          /* index in rank j's shard  */
            if (k >= numel[t]) { out[e] = 0.0f; continue; }
            int64_t src = (layout == ORC_GRADS_FULL) ? L.full_off[t] + k : e;
            for (int32_t r = 0; r < nd; ++r) vals[r] = load_as_f32(grads[r], src, dtype);
            out[e] = sum_ranks(vals, nd);
        }
    }
    free(vals);
    layout_free(&L);
    return 0;
}

void orc_reduce_values(int64_t n, int32_t nd, const void* vals, int32_t dtype,
                       float* out) {
    float* row = (float*)malloc(sizeof(float) * (size_t)(nd > 0 ? nd : 1));
    if (!row) return;
    for (int64_t i = 0; i < n; ++i) {
        for (int32_t r = 0; r < nd; ++r) row[r] = load_as_f32(vals, i * nd + r, dtype);
        out[i] = sum_ranks(row, nd);
    }
    free(row);
}

/* [ZST] "Stage 2 also partitions gradients": with several micro-batches,
 * each one's reduced shard is added into a running shard-sized sum. */
void orc_accumulate(int64_t n, float* acc, const float* g) {
    for (int64_t i = 0; i < n; ++i) acc[i] = acc[i] + g[i];
}

/* ------------------------------------------------------------------ */
/* Adam on the owned shard ([ZD] section 3 "update"; [ZS3]; [ZST])      */
/* ------------------------------------------------------------------ */

/* Scalars fixed per call: 1-b1 and 1-b2 in fp32; the bias corrections
 * 1-b1^t and 1-b2^t in double, rounded once to fp32; t counts from 1. */
void orc_adam_scalars(float b1, float b2, int64_t step, float* out4) {
    out4[0] = 1.0f - b1;
    out4[1] = 1.0f - b2;
    out4[2] = (float)(1.0 - pow((double)b1, (double)step));
    out4[3] = (float)(1.0 - pow((double)b2, (double)step));
}

/* Kingma & Ba, Algorithm 1, one element:
 *   m <- b1*m + (1-b1)*g ;  v <- b2*v + (1-b2)*g^2
 *   mhat = m/(1-b1^t) ;  vhat = v/(1-b2^t)
 *   p <- p - lr*mhat/(sqrt(vhat) + eps)
 * and the bf16 working copy is refreshed from the new fp32 master. */
static void adam_one(float* p, float* m, float* v, uint16_t* w, float g,
                     float lr, float b1, float b2, float eps, const float* sc) {
    float omb1 = sc[0], omb2 = sc[1], bc1 = sc[2], bc2 = sc[3];
    float m_new = b1 * (*m) + omb1 * g;
    float v_new = b2 * (*v) + omb2 * (g * g);
    float mhat = m_new / bc1;
    float vhat = v_new / bc2;
    float denom = sqrtf(vhat) + eps;
    float update = (lr * mhat) / denom;
    float p_new = *p - update;
    *m = m_new;
    *v = v_new;
    *p = p_new;
    *w = orc_bf16_rne(p_new);
}

void orc_adam_elems(int64_t n, float* master, float* m, float* v,
                    uint16_t* work, const float* g,
                    float lr, float b1, float b2, float eps, int64_t step) {
    float sc[4];
    orc_adam_scalars(b1, b2, step, sc);
    for (int64_t i = 0; i < n; ++i)
        adam_one(&master[i], &m[i], &v[i], &work[i], g[i], lr, b1, b2, eps, sc);
}

/* Each rank updates only its own slice; pad elements are not parameters and
 * are left as they are. */
int orc_adam(int32_t T, const int64_t* numel, int32_t nd, int32_t j,
             float* master, float* m, float* v, uint16_t* work, const float* g,
             float lr, float b1, float b2, float eps, int64_t step) {
    if (j < 0 || j >= nd || step < 1) return -1;
    layout_t L;
    if (layout_make(T, numel, nd, &L) != 0) return -1;
    float sc[4];
    orc_adam_scalars(b1, b2, step, sc);
    for (int32_t t = 0; t < T; ++t) {
        int64_t s = L.shard_len[t];
        for (int64_t i = 0; i < s; ++i) {
            int64_t k = (int64_t)j * s + i;
            if (k >= numel[t]) continue;
            int64_t e = L.shard_off[t] + i;
            adam_one(&master[e], &m[e], &v[e], &work[e], g[e], lr, b1, b2, eps, sc);
        }
    }
    layout_free(&L);
    return 0;
}

/* ------------------------------------------------------------------ */
/* Gather ([ZD] section 3; [ZS3] on-demand fetch; [ZST] stage 3)       */
/* ------------------------------------------------------------------ */

/* All-gather rebuilds the full parameter: element k of tensor t lives in rank
 * r = k / s_t at position k - r*s_t of that rank's slice; pad is dropped. */
int orc_gather(int32_t T, const int64_t* numel, int32_t nd, int32_t t,
               const void* src, int32_t dtype, void* out) {
    if (t < 0 || t >= T) return -1;
    if (dtype != ORC_F32 && dtype != ORC_BF16) return -1;
    layout_t L;
    if (layout_make(T, numel, nd, &L) != 0) return -1;
    int64_t s = L.shard_len[t];
    for (int64_t k = 0; k < numel[t]; ++k) {
        int64_t r = k / s;
        int64_t idx = r * L.S + L.shard_off[t] + (k - r * s);
        if (dtype == ORC_BF16) ((uint16_t*)out)[k] = ((const uint16_t*)src)[idx];
        else ((float*)out)[k] = ((const float*)src)[idx];
    }
    layout_free(&L);
    return 0;
}
