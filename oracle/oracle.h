/*
 * oracle.h -- plain CPU oracle for the per-rank hot path of ZeRO-3
 * intra-layer partitioning (flatten + pad + 1D shard, reduce of every rank's
 * gradient into the owned shard, mixed-precision Adam on the shard, gather of
 * the full unpadded parameter).
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may include, link,
 * load or call this code: only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark use it. It shares no source, header, table or
 * helper with the HIP library.
 *
 * Pages this follows (cited by title and section):
 *   [ZD]  "The ZeRO-3 Diagram Most People Remember Is Wrong"
 *   [ZS3] "ZeRO Stage 3: Parameter Partitioning"
 *   [ZST] "ZeRO Stages: Sharding Optimizer State, Gradients, and Parameters"
 * The Adam update itself is not printed on the pages; the oracle takes the
 * textbook definition (Kingma & Ba, "Adam: A Method for Stochastic
 * Optimization", Algorithm 1).
 *
 * Conventions
 *   nd        number of data-parallel ranks (N_d)
 *   numel[t]  element count of tensor t, flattened row-major
 *   dtype     ORC_F32 (fp32 values) or ORC_BF16 (raw bf16 bit patterns, uint16)
 *   All index tables are int64. Arrays named *_off hold T+1 entries
 *   (exclusive prefix sums; the last entry is the total).
 *   "All ranks" state arrays hold nd*S elements with rank r at [r*S, (r+1)*S).
 */
#ifndef ZSP_ORACLE_H
#define ZSP_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORC_F32 = 0, ORC_BF16 = 1 };
enum { ORC_GRADS_FULL = 0, ORC_GRADS_SHARD = 1 };

/* Padding so that numel + pad divides evenly by nd ([ZD] section 2, step 3). */
int64_t orc_pad(int64_t numel, int32_t nd);

/* Per-tensor layout tables ([ZD] section 2; [ZST] "What stage 1 partitions").
 * Outputs: pad[T], shard_len[T], full_off[T+1], shard_off[T+1], flat_off[T+1];
 * *S = elements one rank owns. Returns 0, or -1 on bad arguments. */
int orc_layout(int32_t T, const int64_t* numel, int32_t nd,
               int64_t* pad, int64_t* shard_len,
               int64_t* full_off, int64_t* shard_off, int64_t* flat_off,
               int64_t* S);

/* Model-state bytes a rank holds: 16 bytes per owned element
 * ([ZS3] equation M_Stage3). */
int64_t orc_model_state_bytes(int64_t shard_elems);

/* Model-state bytes one rank holds under ZeRO stage `stage` (0 = plain data
 * parallelism, every term replicated) for psi parameters of which the rank
 * owns shard_elems ([ZST] stage 1 and stage 2 sections; [ZS3] M_Stage3):
 * 16-bit parameters (2 B), gradients of grad_bytes (2 in [ZS3]'s 16-byte
 * budget, 4 in [ZST]'s 18-byte one) and the fp32 master + Adam moments
 * (12 B). Stage 1 shards the optimizer bytes, stage 2 the gradients too,
 * stage 3 everything. Returns -1 for a stage outside 0..3. */
int64_t orc_stage_state_bytes(int32_t stage, int64_t psi, int64_t shard_elems,
                              int32_t grad_bytes);

/* Elements one rank sends per step under ZeRO stage `stage` for n
 * parameters over p ranks, from the collectives each stage runs ([ZST]
 * stage sections and "Communication volume compared"): a reduce-scatter or
 * an all-gather moves n(p-1)/p per rank, an all-reduce is the two in turn.
 * Stage 0 all-reduces gradients; 1 all-reduces them and all-gathers the
 * updated parameters; 2 reduce-scatters and all-gathers; 3 reduce-scatters
 * and gathers the parameters twice (forward and backward). -1 if invalid. */
double orc_stage_comm_elems(int32_t stage, int64_t n, int32_t p);

/* fp32 -> bf16, round to nearest, ties to even (bit pattern). */
uint16_t orc_bf16_rne(float x);
void orc_bf16_rne_array(int64_t n, const float* x, uint16_t* out);

/* Copy-in: split every flattened, padded tensor of `flat` (tensor t at
 * flat_off[t], unpadded) into the shards of ranks [rank_lo, rank_hi).
 * Outputs hold (rank_hi-rank_lo)*S elements. Pads are +0.0 everywhere;
 * m = v = +0.0. Returns 0 or -1. */
int orc_partition(int32_t T, const int64_t* numel, int32_t nd,
                  int32_t rank_lo, int32_t rank_hi,
                  const void* flat, int32_t dtype,
                  float* master, uint16_t* work, float* m, float* v);

/* Reduce into rank j's shard: out[e] = sum over r = 0..nd-1, in that order,
 * of rank r's gradient element, in fp32. grads[r] is rank r's full padded
 * gradient (ORC_GRADS_FULL, tensor t at full_off[t]) or the S-element chunk
 * rank r sends to rank j (ORC_GRADS_SHARD). Pad positions give +0.0 and are
 * never read. Returns 0 or -1. */
int orc_reduce(int32_t T, const int64_t* numel, int32_t nd, int32_t j,
               const void* const* grads, int32_t dtype, int32_t layout,
               float* out);

/* Same sum on values already gathered: vals is n x nd (rank index fastest). */
void orc_reduce_values(int64_t n, int32_t nd, const void* vals, int32_t dtype,
                       float* out);

/* acc[i] = acc[i] + g[i] for i < n (micro-batch accumulation of reduced
 * slices, [ZST] "Stage 2 also partitions gradients"). */
void orc_accumulate(int64_t n, float* acc, const float* g);

/* Host-side step scalars: out = {1-b1, 1-b2, 1-b1^step, 1-b2^step}. */
void orc_adam_scalars(float b1, float b2, int64_t step, float* out4);

/* Adam on n elements, then work = bf16_rne(master). */
void orc_adam_elems(int64_t n, float* master, float* m, float* v,
                    uint16_t* work, const float* g,
                    float lr, float b1, float b2, float eps, int64_t step);

/* Adam on rank j's shard (S elements; pads untouched). Returns 0 or -1. */
int orc_adam(int32_t T, const int64_t* numel, int32_t nd, int32_t j,
             float* master, float* m, float* v, uint16_t* work, const float* g,
             float lr, float b1, float b2, float eps, int64_t step);

/* Gather: rebuild tensor t (numel[t] elements, pads dropped) from the shards
 * of all nd ranks; src holds nd*S elements of `dtype`. Returns 0 or -1. */
int orc_gather(int32_t T, const int64_t* numel, int32_t nd, int32_t t,
               const void* src, int32_t dtype, void* out);

#ifdef __cplusplus
}
#endif

#endif
