/*
 * zsp.h -- C ABI of libzsp, the per-rank hot path of ZeRO-3 intra-layer
 * partitioning on one MI355X (gfx950): N_d data-parallel ranks live as
 * "virtual ranks" in one GPU's memory and every exchange between them is a
 * local HIP kernel.
 *
 * Pages the operations follow (cited by title and section):
 *   [ZD]  "The ZeRO-3 Diagram Most People Remember Is Wrong"
 *         section 2 (flatten, pad, contiguous slice per rank) and section 3
 *         (AllGather before compute, ReduceScatter of gradients, optimizer
 *         updates the local shard)
 *   [ZS3] "ZeRO Stage 3: Parameter Partitioning" (on-demand fetch steps,
 *         equation M_Stage3 and its 7B / 64-GPU example)
 *   [ZST] "ZeRO Stages: Sharding Optimizer State, Gradients, and Parameters"
 *         ("What stage 1 partitions": rank i owns [i*N/P, (i+1)*N/P);
 *          "Stage 2 also partitions gradients": reduce-scatter, shard-sized
 *          gradient buffer, each micro-batch's reduced shard summed into a
 *          running one)
 * The Adam update is the textbook one (Kingma & Ba, Algorithm 1), which the
 * pages name without printing.
 *
 * Terms
 *   nd            number of data-parallel ranks (N_d), 1..ZSP_MAX_RANKS
 *   numel[t]      element count of parameter t, flattened row-major
 *   pad[t]        (nd - numel[t] % nd) % nd
 *   shard_len[t]  (numel[t] + pad[t]) / nd   -- s_t
 *   S             sum of shard_len over all parameters: elements one rank owns
 *   full_off[t]   sum_{u<t} (numel[u] + pad[u])   (full padded layout)
 *   shard_off[t]  sum_{u<t} shard_len[u]          (a rank's shard layout)
 *   flat_off[t]   sum_{u<t} numel[u]              (unpadded concatenation)
 *   total_numel   sum of numel over all parameters
 *   Rank r owns elements [r*s_t, (r+1)*s_t) of padded parameter t and stores
 *   them at shard_off[t] of its shard; positions >= numel[t] are pad.
 *
 * Memory and ownership
 *   The caller allocates and owns every device buffer (parameters, gradients,
 *   optimizer state, accumulator, gather outputs, schedule arenas). A plan
 *   owns its host tables, the device copies of its offset tables (allocated
 *   in zsp_bind_state), the staging slots of long zsp_gather_many lists
 *   (allocated when such a list first needs them; a prepared list,
 *   zsp_gather_list_create, owns memory of its own) and, from its first
 *   checkpoint save or load, the checkpoint staging (pinned host chunks,
 *   streams, events); zsp_destroy frees them. The other hot-path calls
 *   (reduce, Adam, the range and single gathers, schedule acquire and
 *   release) allocate nothing; checkpoint calls also use host memory for
 *   their own duration. The reduce, Adam, range and single gather calls,
 *   zsp_gather_list_run, and zsp_gather_many on lists of at most 64
 *   parameters, only check
 *   arguments and launch kernels (no host wait, no copy, no memset), so they
 *   can be captured into a HIP graph; Adam's scalars (lr, betas, eps and the
 *   step's bias corrections) are kernel arguments, so a replay repeats the
 *   step it was captured with.
 *   Every device pointer must be 16-byte aligned (torch allocations are).
 *   State arrays bound for all ranks hold nd*S elements, rank r at
 *   [r*S, (r+1)*S); bound for one rank j they hold that rank's S elements.
 *
 * Streams
 *   Every call that touches the device enqueues its kernels on `stream` (a
 *   hipStream_t; NULL is the default stream) and returns without waiting.
 *   The caller keeps buffers alive until the stream has run them. The plan is
 *   tied to the device that was current at zsp_bind_state; calls made with
 *   another device current fail with ZSP_ESTATE.
 *
 * Errors
 *   Arguments are checked before anything is enqueued; a bad argument returns
 *   a negative zsp_status and enqueues nothing. A failed kernel launch returns
 *   ZSP_EHIP. zsp_last_error() gives a message for the calling thread's most
 *   recent failure. Values are not checked: NaN and Inf propagate.
 *
 * Threads
 *   The reduce, Adam and gather calls (whole-model and _params forms, list
 *   gathers, prepared-list create and run) and zsp_load_params only read
 *   the plan (zsp_gather_many takes the plan's staging slots under a lock
 *   of their own): several threads may issue them on one plan at once, e.g.
 *   one thread per rank, each on its own stream (work that writes the same
 *   state at the same time is the caller's race, as for any two kernels).
 *   zsp_bind_state, the checkpoint calls and zsp_destroy change the plan
 *   and must not overlap any other call on it.
 *   A schedule's calls must not overlap one another; other schedules and
 *   the read-only calls above may run beside them. Different plans are
 *   independent.
 */
#ifndef ZSP_H
#define ZSP_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct zsp_plan zsp_plan;
typedef struct zsp_sched zsp_sched;
typedef struct zsp_gather_list zsp_gather_list;

typedef enum {
    ZSP_OK = 0,
    ZSP_EINVAL = -1, /* bad argument: null/misaligned pointer, bad rank, dtype, ... */
    ZSP_ERANGE = -2, /* index or size out of the supported range */
    ZSP_ENOMEM = -3, /* host or device allocation for the plan's tables failed */
    ZSP_EHIP = -4,   /* a HIP runtime call or kernel launch failed */
    ZSP_ESTATE = -5, /* call not valid in the plan's current binding/device */
    ZSP_EIO = -6     /* checkpoint file missing, unreadable, corrupt or of another model */
} zsp_status;

typedef enum { ZSP_F32 = 0, ZSP_BF16 = 1 } zsp_dtype;

typedef enum {
    ZSP_GRADS_FULL = 0,  /* grads[r]: rank r's full padded gradient, tensor t at full_off[t] */
    ZSP_GRADS_SHARD = 1  /* grads[r]: indexed like the bound state arrays (see below) */
} zsp_grad_layout;

typedef enum {
    ZSP_SRC_WORK = 0,    /* bf16 working copy of the parameters */
    ZSP_SRC_MASTER = 1,  /* fp32 master parameters */
    ZSP_SRC_ACC = 2      /* fp32 gradient accumulator: each rank's reduced slice */
} zsp_source;

#define ZSP_ALL_RANKS (-1)
#define ZSP_MAX_RANKS 256

/* partition(param list, N_d) -- [ZD] section 2; [ZST] "What stage 1
 * partitions". Builds the per-parameter layout tables for n_params
 * parameters of numel[0..n_params) elements split over n_d ranks. Host only:
 * touches no device. n_params >= 1, numel[t] >= 0, 1 <= n_d <= ZSP_MAX_RANKS.
 * On success *out receives a new plan (free with zsp_destroy). */
zsp_status zsp_partition(const int64_t* numel, int32_t n_params, int32_t n_d,
                         zsp_plan** out);

/* Release the plan, its host tables and its device tables. NULL is ignored.
 * The caller must make sure no enqueued work still reads the tables. */
void zsp_destroy(zsp_plan* plan);

/* Sizes of the plan. Any output pointer may be NULL.
 *   shard_elems  S
 *   total_padded sum of numel+pad (elements of one full-layout gradient)
 *   model_state_bytes_per_rank  16*S: 16-bit param + 16-bit grad + fp32
 *     master + fp32 m + fp32 v per owned element ([ZS3] equation M_Stage3).
 * total_numel and flat_off[t] (see Terms) follow from the numel list. */
zsp_status zsp_plan_info(const zsp_plan* plan, int64_t* shard_elems, int64_t* total_padded,
                         int64_t* model_state_bytes_per_rank);

/* Layout of parameter t (0 <= t < n_params). Any output pointer may be NULL.
 * full_off: its offset in a full-layout gradient; shard_off: its slot's
 * offset in each rank's shard. */
zsp_status zsp_plan_tensor(const zsp_plan* plan, int32_t t, int64_t* numel, int64_t* pad,
                           int64_t* shard_len, int64_t* full_off, int64_t* shard_off);

/* Bind the caller-owned optimizer state and build the device tables.
 *   rank_or_all = ZSP_ALL_RANKS: every array holds n_d*S elements (all ranks
 *     resident on this GPU); every rank-taking call may name any rank or all.
 *   rank_or_all = j: every array holds rank j's S elements only; calls must
 *     name rank j, and gathers are not possible (ZSP_ESTATE).
 *   master, m, v: fp32; work: bf16 bit patterns; grad_acc: fp32 accumulator
 *     or NULL (then accumulate/use_acc calls fail with ZSP_ESTATE).
 * Allocates the device tables (setup path): 40 bytes per bound piece (one
 * rank's slice of one parameter) and 4 bytes per 512 elements of the bound
 * state; an all-rank binding adds the gather's 16 bytes per piece, 36 bytes
 * per 512 elements of the unpadded parameters and 32 bytes per parameter.
 * Rebinding replaces the previous binding. */
zsp_status zsp_bind_state(zsp_plan* plan, int32_t rank_or_all, float* master, float* m,
                          float* v, uint16_t* work, float* grad_acc);

/* Copy-in ([ZD] section 2, steps 1-4): split the unpadded parameters into the
 * bound ranks' shards. flat_params holds total_numel elements of `dtype`,
 * parameter t at flat_off[t]. Writes master = fp32(x), work = x (bf16 input)
 * or its round-to-nearest-even bf16 (fp32 input), m = v = 0, and +0 at every
 * pad position of all four arrays. */
zsp_status zsp_load_params(zsp_plan* plan, const void* flat_params, zsp_dtype dtype,
                           void* stream);

/* reduce_shard(rank, grads[N_d]) -- ReduceScatter restricted to the owned
 * slice ([ZD] section 3; [ZST] "Stage 2 also partitions gradients").
 * For each owned non-pad element: red = sum over r = 0..n_d-1, in rank
 * order, of fp32(grads[r][...]), one fp32 addition at a time starting from
 * rank 0's value. Writes grad_acc = red (accumulate = 0) or
 * grad_acc = grad_acc + red (accumulate = 1); pad positions of grad_acc are
 * set to +0. grads: n_d device pointers (host array) of `dtype`.
 *   ZSP_GRADS_FULL : grads[r] holds total_padded elements; the element of
 *                    parameter t at padded index k is at full_off[t] + k.
 *   ZSP_GRADS_SHARD: grads[r] is the chunk rank r sends to the owners, in the
 *                    bound arrays' indexing: S elements for a one-rank
 *                    binding, n_d*S (owner j at j*S) for an all-rank one.
 * Pad positions of grads are never read. rank_or_all: a rank or
 * ZSP_ALL_RANKS (all-rank binding only). */
zsp_status zsp_reduce_shard(zsp_plan* plan, int32_t rank_or_all, const void* const* grads,
                            zsp_dtype dtype, zsp_grad_layout layout, int32_t accumulate,
                            void* stream);

/* adam_step(shard, lr, beta1, beta2, eps, step) -- the optimizer updates the
 * local shard ([ZD] section 3; [ZS3] on-demand fetch, last step; [ZST]).
 * Uses grad_acc as the gradient. For each owned non-pad element, in fp32 with
 * one rounding per operation, in this order:
 *   m = beta1*m + (1-beta1)*g ;  v = beta2*v + (1-beta2)*(g*g)
 *   mh = m/(1-beta1^step) ;  vh = v/(1-beta2^step)
 *   master = master - (lr*mh)/(sqrt(vh) + eps) ;  work = bf16_rne(master)
 * 1-beta is computed in fp32; 1-beta^step in double and rounded once to
 * fp32. Pad positions are not touched. step >= 1. */
zsp_status zsp_adam_step(zsp_plan* plan, int32_t rank_or_all, float lr, float beta1,
                         float beta2, float eps, int64_t step, void* stream);

/* The hot path: reduce_shard and adam_step fused in one pass. g = red
 * (use_acc = 0) or g = grad_acc + red (use_acc = 1, the last micro-batch of
 * an accumulation window); the reduced gradient stays in registers and
 * grad_acc is not written. Same arithmetic, bit for bit, as reduce_shard
 * followed by adam_step. */
zsp_status zsp_reduce_adam_step(zsp_plan* plan, int32_t rank_or_all,
                                const void* const* grads, zsp_dtype dtype,
                                zsp_grad_layout layout, int32_t use_acc, float lr,
                                float beta1, float beta2, float eps, int64_t step,
                                void* stream);

/* The three calls above restricted to the parameters [first_param,
 * first_param + n_params): only those parameters' slots of each rank the
 * call names are read or written; every other slot, the accumulator's
 * included, is untouched. This is the reduce-scatter of one layer during
 * backward ([ZD] section 6: gradient reduce-scatters appear during backward;
 * [ZS3]: after a layer's backward its gradients go to the ranks owning
 * them), or the update of one layer. grads[] are the same whole-model
 * buffers as above. Each rank's slots of a parameter range are one
 * contiguous span, so the call is one launch per rank (one launch for every
 * parameter). ZSP_ERANGE if the range is empty or outside [0, n_params). */
zsp_status zsp_reduce_shard_params(zsp_plan* plan, int32_t rank_or_all, int32_t first_param,
                                   int32_t n_params, const void* const* grads, zsp_dtype dtype,
                                   zsp_grad_layout layout, int32_t accumulate, void* stream);
zsp_status zsp_adam_step_params(zsp_plan* plan, int32_t rank_or_all, int32_t first_param,
                                int32_t n_params, float lr, float beta1, float beta2, float eps,
                                int64_t step, void* stream);
zsp_status zsp_reduce_adam_step_params(zsp_plan* plan, int32_t rank_or_all, int32_t first_param,
                                       int32_t n_params, const void* const* grads,
                                       zsp_dtype dtype, zsp_grad_layout layout, int32_t use_acc,
                                       float lr, float beta1, float beta2, float eps,
                                       int64_t step, void* stream);

/* gather(param_id) -- AllGather of a full parameter just before compute
 * ([ZD] section 3; [ZS3] on-demand fetch, step 2; [ZST] "Stage 3
 * partitions parameters"). Writes numel[param_id] elements to `out`, pad
 * dropped: out[k] = src_r[shard_off[t] + k - r*s_t] with r = k / s_t.
 * src = ZSP_SRC_WORK (bf16 out), ZSP_SRC_MASTER (fp32 out) or ZSP_SRC_ACC
 * (fp32 out, needs an accumulator bound): gathering the reduced gradient
 * slices completes an all-reduce of the gradients, the reduction stage 1
 * keeps ([ZST] "What stage 1 partitions": gradients arrive complete on
 * every rank, each rank updates its own slice); pad slots are dropped as
 * for parameters. Needs an all-rank binding. */
zsp_status zsp_gather(zsp_plan* plan, int32_t param_id, zsp_source src, void* out,
                      void* stream);

/* Gather of the consecutive parameters [first_param, first_param +
 * n_params) -- one layer's worth, e.g. -- in one launch ([ZD] section 3:
 * each layer's parameters are all-gathered just before it runs). `out`
 * receives them back to back, unpadded: parameter t at flat_off[t] -
 * flat_off[first_param]. ZSP_ERANGE if the range is empty or outside
 * [0, n_params). The per-layer schedule below uses this gather. */
zsp_status zsp_gather_range(zsp_plan* plan, int32_t first_param, int32_t n_params,
                            zsp_source src, void* out, void* stream);

/* gather(param_id) for a list of parameters: ids[0..n) in any order
 * (repeats allowed), parameter ids[i] into its own output outs[i]
 * (numel[ids[i]] elements, unpadded, as zsp_gather writes them). This is
 * the all-gather of a bucket of parameters, e.g. the module about to run
 * ([ZD] section 3: a module's full parameters are gathered just before its
 * forward and again before its backward; section 8: gathers go out in
 * buckets of parameters). ids and outs are host arrays, read during the
 * call; every outs[i] of a non-empty parameter must be a 16-byte aligned
 * device pointer (NULL is allowed for empty ones); outputs must not
 * overlap one another or the bound state. n = 0 does nothing.
 *   Lists of at most 64 non-empty parameters: one launch, nothing staged.
 *   Longer lists: their entries (16 bytes per parameter plus 4 bytes per
 *   32768 output elements) go to the device through one of four staging
 *   slots the plan keeps (a copy kernel reads them from the slot's pinned
 *   host buffer), then two launches per chunk of records. A slot is allocated
 *   (pinned host and device memory) the first time a list needs more room
 *   than it has -- the only allocation of any gather call -- and is refilled
 *   only after the gathers of its previous use have run: the call waits on
 *   the host when four staged gathers are still in flight. Each slot holds
 *   the records of at most 2^19 tiles of 512 elements (16 MiB); longer
 *   lists go in several pairs of launches.
 * Errors: ZSP_ERANGE for an id outside [0, n_params) or a list of 2^31
 * tiles or more; ZSP_EINVAL for NULL arrays with n > 0, a NULL or
 * misaligned output, or n < 0; ZSP_ESTATE without an all-rank binding;
 * ZSP_ENOMEM if a staging slot cannot grow. Needs an all-rank binding. */
zsp_status zsp_gather_many(zsp_plan* plan, const int32_t* ids, int32_t n, zsp_source src,
                           void* const* outs, void* stream);

/* zsp_gather_many for callers that cannot allocate (tight serving loops,
 * harnesses that forbid allocation, and code under HIP graph capture for
 * lists of at most 64 non-empty parameters, which are one kernel launch):
 * the same arguments, checks and results, but nothing is allocated, on the
 * device or the host. A longer list's staging copy reads a host buffer that
 * the next call refills, so a captured copy would replay stale entries:
 * capture such lists as a prepared list (zsp_gather_list_run) instead.
 * A long list (more than 64 non-empty parameters) is staged
 * in a fixed device array the library holds on every GPU it runs on from
 * load to process end (9.25 MiB): its entries and coarse index are copied
 * there from a static host buffer, then the same two kernels run. Limits:
 * at most 65536 non-empty parameters and 2^22 tiles of 512 elements (2^31
 * elements) per call, else ZSP_ERANGE; longer lists than 2^18 tiles run in
 * several pairs of launches. The array keeps the last call's contents and
 * every call on a GPU shares it: calls on one stream run in order, but
 * calls that overlap on one GPU (other streams or threads) race. The array's
 * address is taken at an all-rank zsp_bind_state (or the first call) on
 * each device. Lists of at most 64 non-empty parameters touch no staging
 * at all, as in zsp_gather_many. */
zsp_status zsp_gather_many_noalloc(zsp_plan* plan, const int32_t* ids, int32_t n,
                                   zsp_source src, void* const* outs, void* stream);

/* A list gather prepared once and run many times: the same bucket into the
 * same outputs every step ([ZD] section 3: a module's parameters are
 * gathered before its forward and again before its backward, every step;
 * section 8: gathers go out in buckets). zsp_gather_list_create takes the
 * arguments of zsp_gather_many, with the same checks and errors, and keeps
 * what a run needs: for a list of more than 64 non-empty parameters, its
 * per-tile records (32 bytes per 512 output elements, plus 16 bytes per
 * parameter), built on the device once -- create allocates that memory,
 * enqueues the build on `stream` and waits for it before returning
 * (ZSP_ENOMEM if the allocation fails). Lists of at most 64 keep their
 * entries on the host and run as zsp_gather_many's one launch.
 *   zsp_gather_list_run enqueues the gather on `stream`: one launch, no
 * copy, no allocation, no host wait (capturable into a HIP graph). It reads
 * the source named at create from the plan's current binding, so the list
 * stays valid when state is bound again on the same device; the outputs
 * named at create must stay allocated while runs may be in flight.
 * ZSP_ESTATE if the plan has no all-rank binding now, is bound on another
 * device than at create, or the source is the accumulator and none is
 * bound; ZSP_EINVAL for a NULL list.
 *   zsp_gather_list_destroy frees the list (NULL is a no-op); runs must have
 * finished. A list refers to its plan, which must outlive it. */
zsp_status zsp_gather_list_create(zsp_plan* plan, const int32_t* ids, int32_t n,
                                  zsp_source src, void* const* outs, void* stream,
                                  zsp_gather_list** list);
zsp_status zsp_gather_list_run(zsp_gather_list* list, void* stream);
void zsp_gather_list_destroy(zsp_gather_list* list);

/* ---- Per-layer gather schedule with prefetch ------------------------------
 * [ZS3] on-demand fetch list (gather layer l before its computation, discard
 * after) and prefetch paragraph (gather layer l+1 while layer l computes);
 * [ZST] "Stage 3 partitions parameters" (gather before forward, again before
 * backward, release after use; prefetch depth trades memory for latency).
 * A schedule visits groups of consecutive parameters (one layer each) in a
 * fixed order of positions. Position p is gathered into slot p mod (D+1) of
 * a caller-owned device arena, D = prefetch depth; with D > 0 the gathers of
 * positions up to p+D run on a gather stream of the caller's while the
 * compute stream works on p. All ordering is by HIP events (no host waits):
 * a gather into a slot follows the release of the slot's previous position,
 * a pass's first gathers follow what the compute stream did before position
 * 0's acquire (e.g. the optimizer step), and the compute stream's work after
 * an acquire follows that position's gather. D = 0 gathers on the compute
 * stream in line. The plan must outlive the schedule. */

/* Build a schedule over `plan` (host only). Group g is the parameters
 * [group_first[g], group_first[g] + group_count[g]); order[p] is the group
 * of position p, 0 <= p < n_steps. 0 <= depth <= 64 (depths beyond
 * n_steps - 1 act as n_steps - 1). *arena_bytes receives the device bytes
 * zsp_sched_bind needs: (D+1) slots, each the largest group's gathered size
 * (2 B per element for ZSP_SRC_WORK, 4 for ZSP_SRC_MASTER) rounded up to
 * 256 B. Every gather is zsp_gather_range's kernel. */
zsp_status zsp_sched_create(zsp_plan* plan, int32_t n_groups, const int32_t* group_first,
                            const int32_t* group_count, int32_t n_steps, const int32_t* order,
                            int32_t depth, zsp_source src, int64_t* arena_bytes,
                            zsp_sched** out);

/* Attach the arena (caller-owned device memory of at least *arena_bytes,
 * 256-byte aligned) and the gather stream (required when D > 0; a stream
 * other than the compute stream, at default priority). Needs an all-rank
 * binding of the plan, on the current device. Creates the schedule's HIP
 * events; a later bind replaces them and restarts at position 0. */
zsp_status zsp_sched_bind(zsp_sched* sched, void* arena, int64_t arena_bytes,
                          void* gather_stream);

/* Acquire position `position` for work on `compute_stream`: issue any
 * gathers not yet issued up to position + D, order the compute stream after
 * this position's gather, and return in *params the device address of its
 * group: parameter t at flat_off[t] - flat_off[first] elements, unpadded.
 * Positions are acquired in order 0..n_steps-1, each released before the
 * next is acquired; after the last, the next pass starts at 0. Otherwise
 * ZSP_ESTATE. */
zsp_status zsp_sched_acquire(zsp_sched* sched, int32_t position, void* compute_stream,
                             void** params);

/* Release the held position: every use of its slot must already be enqueued
 * on `compute_stream`; the slot may be overwritten once that work is done. */
zsp_status zsp_sched_release(zsp_sched* sched, int32_t position, void* compute_stream);

typedef enum {
    ZSP_ENGINE_KERNEL = 0, /* the gather kernel (zsp_gather_range's), on the CUs */
    ZSP_ENGINE_COPY = 1    /* the DMA copy engines: no compute units */
} zsp_gather_engine;

/* What runs the schedule's gathers ([ZS3] prefetch paragraph: the next
 * layer's gather should overlap the current layer's computation; a gather
 * kernel competes with that computation for the CUs, the copy engines do
 * not). ZSP_ENGINE_COPY issues one device-to-device copy per rank's slice
 * of each parameter (n_d per parameter) on the stream the kernel would run
 * on, ordered by the same events. Takes effect at the next zsp_sched_bind:
 * a bound schedule is unbound (ZSP_ESTATE until bound again); ZSP_ESTATE
 * while a position is held. */
zsp_status zsp_sched_set_engine(zsp_sched* sched, zsp_gather_engine engine);

/* Abandon the current pass; the next acquire is position 0. Gathers already
 * issued still complete in stream order before any later one. */
zsp_status zsp_sched_reset(zsp_sched* sched);

/* Effective depth, slot count and slot stride in bytes. Host only. */
zsp_status zsp_sched_info(const zsp_sched* sched, int32_t* depth, int32_t* slots,
                          int64_t* slot_bytes);

/* Free the schedule and its events (the arena stays the caller's). Work
 * already enqueued is unaffected. NULL is a no-op. */
void zsp_sched_destroy(zsp_sched* sched);

/* ---- Sharded checkpoint, resume and reshard ------------------------------
 * [ZST] "Where the shards live and what happens on failure": each rank
 * writes its own shard set together with the layout it was cut with; loading
 * under a different rank count reshuffles the shards; the consistent point is
 * between steps (the gradient accumulator is not saved).
 * A checkpoint is a directory holding one file per rank,
 * "rank-<r>-of-<n_d>.zsp": a header (magic "ZSPCKPT1", n_d, rank, number of
 * parameters, S, step), the numel list, master[S], m[S], v[S] (fp32), work[S]
 * (bf16 bits), and the XXH64 hash (seed 0) of all of it, all little-endian.
 * The directory must exist. */

/* Write rank `rank`'s shard set from host arrays of S elements each. Host
 * only. Files are written under a temporary name and renamed. */
zsp_status zsp_checkpoint_write_host(const zsp_plan* plan, int32_t rank, const char* dir,
                                     int64_t step, const float* master, const float* m,
                                     const float* v, const uint16_t* work);

/* Read rank `rank`'s shard set for this plan's layout into host arrays of S
 * elements each; *step receives the saved step. If the checkpoint was written
 * with another rank count, every one of its rank files is read and the shard
 * is rebuilt for this plan (element k of parameter t comes from old rank
 * k / s_old, pads are +0): a reshard, bit-exact. The saved numel list must
 * equal the plan's, else ZSP_EIO; a file whose S differs is refused before
 * anything is written to the arrays, otherwise on error their contents are
 * unspecified. Host only. */
zsp_status zsp_checkpoint_read_host(const zsp_plan* plan, int32_t rank, const char* dir,
                                    int64_t* step, float* master, float* m, float* v,
                                    uint16_t* work);

/* Save the bound state of one rank or of every bound rank
 * (ZSP_ALL_RANKS) to `dir`. The copies follow everything already enqueued
 * on `stream` (an event taken on it orders the library's own copy streams);
 * returns after the files are written. Up to 16 files are written at once,
 * through pinned host chunks the plan keeps until zsp_destroy (32 MiB per
 * file in flight, 512 MiB at most). */
zsp_status zsp_checkpoint_save(zsp_plan* plan, int32_t rank_or_all, const char* dir,
                               int64_t step, void* stream);

/* Load one rank or every bound rank from `dir` into the bound state,
 * resharding if the checkpoint has another rank count; *step receives the
 * saved step. Every file involved is read and checked (header, parameter
 * list, checksum, one common step) before any device write, so a failed
 * load leaves the state untouched. The copies follow everything already
 * enqueued on `stream` and complete before the call returns. Restoring only
 * rank r (e.g. after losing it) leaves the other ranks' state untouched. */
zsp_status zsp_checkpoint_load(zsp_plan* plan, int32_t rank_or_all, const char* dir,
                               int64_t* step, void* stream);

/* Message for the calling thread's most recent failed call ("" if none). */
const char* zsp_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* ZSP_H */
