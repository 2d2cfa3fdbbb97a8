/*
 * ddpsim.h -- C ABI of libddpsim.so: the data-parallel gradient
 * synchronisation hot path (bucket plan, flatten, ring all-reduce with
 * averaging, unflatten, the in-place bucket all-reduce and the reducer that
 * launches it as gradients become ready, the standalone reduce-scatter /
 * all-gather / broadcast, the logarithmic-latency all-reduce schedules and
 * their choice by size, the overlapped step-time model, and the coalesced
 * broadcast of parameters and buffers), with p simulated ranks whose
 * buffers all live in the HBM of one gfx950 GPU.
 *
 * Pages this interface follows, cited by title and section:
 *   [DDP] "PyTorch DDP Deep Dive -- Initialization, Buffer Broadcast, the
 *         Reducer, and the torch.compile Story"
 *   [COL] "Collective Ops From Scratch"
 *   [DP]  "Data parallelism" (zerotofrontier.app, distributed chapter)
 *
 * Conventions for every entry point
 *   - Device memory (rank buffers, gradients, workspace, the plan's device
 *     table) belongs to the caller. The library never allocates or frees
 *     device memory and never synchronises a stream or the device.
 *   - Host arrays passed in (pointer lists, token counts) are read during
 *     the call only; their contents are copied into kernel arguments.
 *   - Work is enqueued on `stream` (0 = the null stream). A fault inside a
 *     kernel surfaces at the caller's next synchronisation, as with any
 *     asynchronous HIP call.
 *   - Every argument is validated before anything is enqueued: an error
 *     return means no work was queued. ddp_last_error() then describes the
 *     failure (thread-local, valid until the next call on that thread).
 *   - "Simulated rank r" is index r of a pointer array of length p,
 *     1 <= p <= DDP_MAX_RANKS. Rank buffers must be 16-byte aligned and must
 *     not overlap one another.
 *   - Element types: DDP_F32 (IEEE binary32) and DDP_BF16 (bfloat16).
 *     Sums are always accumulated in fp32; bf16 results are rounded once,
 *     to nearest even.
 *   - Summation order: for the all-reduce, element i of an n-element buffer
 *     lies in chunk c = i / C with C = ceil(n/p), and its sum is
 *     x_c + x_{c+1} + ... + x_{c+p-1} (ranks mod p) accumulated left to
 *     right, exactly the order in which the ring's reduce-scatter adds the
 *     contributions ([COL] "Ring allreduce in two passes"; [DP] "Ring
 *     all-reduce, derived"). Both ring algorithms produce these bits; the
 *     logarithmic schedules of allreduce_sim have their own fixed order.
 *
 * No C++ exception crosses this boundary.
 */
#ifndef DDPSIM_H
#define DDPSIM_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DDP_MAX_RANKS 64

typedef enum {
  DDP_OK = 0,
  DDP_EINVAL = 1,        /* bad argument (null pointer, bad enum, n < 0, ...) */
  DDP_ERANGE = 2,        /* p, bucket or step index out of range            */
  DDP_EALIGN = 3,        /* a buffer is not 16-byte aligned                 */
  DDP_EALIAS = 4,        /* buffers that must be distinct overlap           */
  DDP_ENOTDIVISIBLE = 5, /* reduce-scatter / all-gather: n % p != 0         */
  DDP_ENOTREADY = 6,     /* plan has no device table (ddp_plan_upload)      */
  DDP_EWORKSPACE = 7,    /* workspace missing or too small                  */
  DDP_EHIP = 8           /* a HIP call failed; ddp_last_error() has detail  */
} ddp_status;

typedef enum { DDP_F32 = 0, DDP_BF16 = 1 } ddp_dtype;

/* Averaging applied to the finished sum: none; divide by p; or divide by
 * the total token count summed over ranks ([DP] "Why averaging gradients is
 * exactly large-batch training"; "Overlapping communication with the
 * backward pass"). The division is one correctly rounded fp32 division by
 * (float)p or (float)(sum of tokens). */
typedef enum {
  DDP_AVG_NONE = 0,
  DDP_AVG_WORLD = 1,
  DDP_AVG_TOKENS = 2
} ddp_avg_mode;

/* DDP_ALGO_FUSED: one kernel reads every rank's buffer once, folds each
 *   element in ring order in registers, and writes the result to every rank.
 * DDP_ALGO_RING: the ring schedule step by step, 2(p-1) launches, each rank
 *   adding (reduce-scatter) or copying (all-gather) its neighbour's chunk in
 *   HBM. Same bits as FUSED. */
typedef enum { DDP_ALGO_FUSED = 0, DDP_ALGO_RING = 1 } ddp_algo;

/* Communication accounting of the logical schedule a call implements
 * ([COL] per-rank byte counter; [DP] "Ring all-reduce, derived"). For the
 * ring all-reduce bytes_sent_per_rank = 2 (p-1) C w with w the wire element
 * size (4: partial sums travel as fp32), which is 2T(p-1)/p for the padded
 * tensor of T bytes. hbm_bytes is what the call's kernels must read plus
 * write in device memory (the algorithmic traffic). */
typedef struct {
  int64_t steps;                /* ring steps or tree rounds            */
  int64_t messages;             /* point-to-point messages              */
  int64_t bytes_sent_per_rank;  /* max over ranks                       */
  int64_t bytes_recv_per_rank;  /* max over ranks                       */
  int64_t total_bytes;          /* sum over all messages                */
  int64_t hbm_bytes;            /* algorithmic device-memory traffic    */
} ddp_comm_stats;

typedef struct ddp_plan ddp_plan;

/* ----------------------------------------------------------------------- */
/* Errors                                                                  */
/* ----------------------------------------------------------------------- */

const char *ddp_strerror(ddp_status status);
/* Detail of the most recent failure on this thread ("" if none). */
const char *ddp_last_error(void);
/* Library version string. */
const char *ddp_version(void);

/* Instrumentation. The next call on this thread of an entry point that
 * launches kernels (flatten / unflatten, the all-reduces and collectives,
 * the coalesced broadcast, and a reducer mark that launches a run) attaches
 * `start` to the dispatch of its first kernel and `stop` to the dispatch of
 * its last kernel (hipExtLaunchKernel semantics), so
 * hipEventElapsedTime(start, stop) is exactly the device time of that
 * call's kernels, with nothing else on the stream in between. Host-only
 * calls (planning, uploads, the models, accessors) leave the request
 * pending. Events are created and owned by the caller (hipEventCreate). The
 * request is consumed by that call even if it fails or launches nothing
 * (n == 0); then the events are not recorded. Pass NULL, NULL to cancel.
 * Errors: DDP_EINVAL if exactly one of the two is NULL. */
ddp_status ddp_time_next_call(hipEvent_t start, hipEvent_t stop);

/* ----------------------------------------------------------------------- */
/* Bucket plan (host)                                                      */
/* ----------------------------------------------------------------------- */

/* Assign parameters to buckets ([DDP] Part 1 "What _ddp_init_helper
 * actually does"; Part 3, the DDPOptimizer's reverse walk; [DP]
 * "Overlapping communication with the backward pass").
 *
 *   numel[i]   element count of parameter i, in registration order (>= 0)
 *   n_params   number of parameters (>= 0)
 *   elem_bytes bytes per element (2 or 4); the plan has one dtype
 *   bucket_cap_bytes, first_bucket_cap_bytes   caps (>= 0); the defaults on
 *              the pages are 25 MiB and 1 MiB
 *
 * Parameters are walked from the last registered to the first. Before a
 * parameter is added, a non-empty open bucket whose byte size has reached
 * its cap is closed. The first bucket's cap is min(first, cap), every
 * later bucket's is `cap`. Inside a bucket, parameters sit in fill order at
 * consecutive element offsets. No bucket is empty; a bucket may overshoot
 * its cap by its last parameter.
 *
 * *out receives a host object owned by the caller, freed with
 * ddp_plan_free. Errors: DDP_EINVAL (null out, negative size or cap,
 * elem_bytes not 2 or 4, n_params < 0). */
ddp_status ddp_bucket_plan(const int64_t *numel, int32_t n_params,
                           int32_t elem_bytes, int64_t bucket_cap_bytes,
                           int64_t first_bucket_cap_bytes, ddp_plan **out);
void ddp_plan_free(ddp_plan *plan);

/* The same bucketing over an explicit walk order: order[k] is the k-th
 * parameter to place (a permutation of 0..n_params-1). DDP rebuilds its
 * buckets once, before the next forward, from the order in which the
 * gradients were observed to become ready in the first backward ([DDP] Part
 * 2, "Step 2: backward": the hook records each ready parameter while a
 * rebuild is due; "_pre_forward" runs the rebuild); pass the order that
 * ddp_reducer_ready_order reports. Bucket 0 (the first filled) has the small
 * cap. Errors: as ddp_bucket_plan, plus DDP_EINVAL when order is NULL or
 * not a permutation. */
ddp_status ddp_bucket_plan_ordered(const int64_t *numel, int32_t n_params,
                                   const int32_t *order, int32_t elem_bytes,
                                   int64_t bucket_cap_bytes,
                                   int64_t first_bucket_cap_bytes,
                                   ddp_plan **out);

/* Buckets for a coalesced broadcast ([DDP] Part 2, the buffer broadcast:
 * tensors are coalesced into buckets capped at 250 MiB by default, each
 * flattened and broadcast as one message): tensors in list order; a bucket
 * is closed before a tensor that would take it past cap_bytes, so no bucket
 * exceeds the cap unless one tensor alone does. elem_bytes 1, 2, 4 or 8
 * (broadcasts copy bytes; one plan per element size). Upload the plan's
 * descriptor table (ddp_plan_upload) before ddp_broadcast_coalesced.
 * Errors: DDP_EINVAL. */
ddp_status ddp_coalesce_plan(const int64_t *numel, int32_t n_tensors,
                             int32_t elem_bytes, int64_t cap_bytes,
                             ddp_plan **out);

int32_t ddp_plan_num_params(const ddp_plan *plan);
int32_t ddp_plan_num_buckets(const ddp_plan *plan);
/* Total elements of bucket b (-1 if b is out of range). */
int64_t ddp_plan_bucket_numel(const ddp_plan *plan, int32_t b);
/* Number of parameters in bucket b (-1 if out of range). */
int32_t ddp_plan_bucket_size(const ddp_plan *plan, int32_t b);
/* Writes bucket b's parameter indices, in fill order, to idx_out (room for
 * ddp_plan_bucket_size(b) entries). */
ddp_status ddp_plan_bucket_params(const ddp_plan *plan, int32_t b,
                                  int32_t *idx_out);
/* Bucket holding parameter i, and its element offset inside that bucket
 * (-1 if i is out of range). */
int32_t ddp_plan_param_bucket(const ddp_plan *plan, int32_t i);
int64_t ddp_plan_param_offset(const ddp_plan *plan, int32_t i);
/* Element count of parameter i as the plan was built with it (-1 if i is
 * out of range): what every rank's gradient of parameter i must hold. */
int64_t ddp_plan_param_numel(const ddp_plan *plan, int32_t i);
/* Bytes per element the plan was built for (-1 for a NULL plan). */
int32_t ddp_plan_elem_bytes(const ddp_plan *plan);

/* Size in bytes of the plan's device-side table: 32 bytes per parameter
 * descriptor, then 4 bytes per tile of 4096 elements naming the tile's
 * descriptor. */
size_t ddp_plan_device_bytes(const ddp_plan *plan);
/* Copy the descriptor table into caller-owned device memory `d_table`
 * (at least ddp_plan_device_bytes bytes, 16-byte aligned) on `stream`, and
 * remember that address for ddp_flatten / ddp_unflatten. The caller keeps
 * d_table alive while the plan is used, and must not free the plan before
 * the copy has completed on `stream`. */
ddp_status ddp_plan_upload(ddp_plan *plan, void *d_table, size_t bytes,
                           hipStream_t stream);

/* ----------------------------------------------------------------------- */
/* Flatten / unflatten                                                     */
/* ----------------------------------------------------------------------- */

/* Copy every gradient of bucket `bucket` into each rank's flat bucket
 * buffer at its plan offset ([DDP] Part 2 "Step 2: backward", the copy into
 * the bucket's slice), dividing each element by prescale_divisor on the way
 * in unless it is 1 (the reducer's pre-divide; fp32 division, bf16 rounded
 * once).
 *
 *   d_grad_ptrs  DEVICE array of p * n_params pointers, rank-major:
 *                d_grad_ptrs[r * n_params + i] is rank r's gradient of
 *                parameter i (numel[i] contiguous elements, any alignment
 *                of the element type)
 *   bucket_bufs  HOST array of p device pointers, each to a 16-byte aligned
 *                buffer of ddp_plan_bucket_numel(bucket) elements
 *   dtype        must match the plan's elem_bytes
 * Errors: DDP_ENOTREADY (no ddp_plan_upload), DDP_ERANGE, DDP_EINVAL,
 * DDP_EALIGN, DDP_EALIAS (bucket buffers overlap). Gradients and bucket
 * buffers must not overlap (not checked: device-resident pointers). */
ddp_status ddp_flatten(const ddp_plan *plan, int32_t bucket, int32_t p,
                       const void *const *d_grad_ptrs,
                       void *const *bucket_bufs, int32_t dtype,
                       float prescale_divisor, hipStream_t stream);

/* Copy each slice of the reduced flat bucket buffers back into the
 * per-parameter gradients ([DDP] Part 2 "Step 3: finalize_backward").
 * Same arguments and errors as ddp_flatten, in the other direction. */
ddp_status ddp_unflatten(const ddp_plan *plan, int32_t bucket, int32_t p,
                         const void *const *bucket_bufs,
                         void *const *d_grad_ptrs, int32_t dtype,
                         hipStream_t stream);

/* ----------------------------------------------------------------------- */
/* Bucket all-reduce in place on the gradients                             */
/* ----------------------------------------------------------------------- */

/* The bucket's flatten, ring all-reduce and unflatten as one pass over the
 * gradients: afterwards every rank's gradients of bucket `bucket` hold
 * exactly the bits that ddp_flatten, then ring_allreduce_sim on the flat
 * buffers (same p, dtype, averaging), then ddp_unflatten would leave there.
 * No flat buffer is materialised: the ring's chunks (ceil(n_b/p) elements
 * of the bucket's flat index space, [COL] "Ring allreduce in two passes")
 * are mapped onto the parameters through the plan ([DDP] Part 2 "Step 2:
 * backward" item 1 and "Step 3: finalize_backward" describe the copies this
 * replaces). Device-memory traffic is 2 p n_b bytes-per-element.
 *
 * Before the first call for a given p, upload the plan's descriptor table
 * for p (each parameter's offset in its bucket and the bucket's ring chunk
 * size for p, then a map from 256-element tiles to descriptors):
 * ddp_plan_segment_bytes(plan, p) bytes of caller-owned device memory
 * (16-byte aligned), filled by ddp_plan_upload_segments on `stream`. The
 * plan keeps the host copy alive; uploading for another p replaces it, and
 * a refused upload leaves the previous table in use. The caller keeps the
 * device memory alive while launches may read it, on any stream.
 *
 *   d_grad_ptrs  DEVICE array of p * n_params gradient addresses, rank-major
 *                (as for ddp_flatten); each gradient must be aligned to its
 *                element size. When every rank's copy of a parameter has the
 *                same offset from a 16-byte boundary the kernel moves 16-byte
 *                vectors, otherwise elements.
 *   avg_mode, tokens, stats   as ring_allreduce_sim.
 * Errors: DDP_ENOTREADY (no descriptor table for this p), DDP_ERANGE,
 * DDP_EINVAL. Gradients of different ranks or parameters must not overlap
 * (not checked here: the addresses are device-resident; the Python
 * binding's grad_pointer_table refuses overlapping gradients). */
size_t ddp_plan_segment_bytes(const ddp_plan *plan, int32_t p);
ddp_status ddp_plan_upload_segments(ddp_plan *plan, int32_t p, void *d_table,
                                    size_t bytes, hipStream_t stream);
ddp_status ddp_allreduce_bucket(const ddp_plan *plan, int32_t bucket,
                                int32_t p, void *const *d_grad_ptrs,
                                int32_t dtype, int32_t avg_mode,
                                const int64_t *tokens, hipStream_t stream,
                                ddp_comm_stats *stats);

/* ddp_allreduce_bucket for the run of buckets [first_bucket,
 * first_bucket + n_buckets) in one kernel launch: the reducer fires every
 * consecutive ready bucket starting at its next bucket ([DDP] Part 2 "Step
 * 2: backward", item 3), and one dispatch for the run avoids a kernel
 * boundary per bucket. Each bucket keeps its own ring chunks; the result is
 * bit-identical to calling ddp_allreduce_bucket on each. Stats add up the
 * buckets' ring schedules. Errors: as ddp_allreduce_bucket, DDP_ERANGE for
 * an empty or out-of-range run. */
ddp_status ddp_allreduce_buckets(const ddp_plan *plan, int32_t first_bucket,
                                 int32_t n_buckets, int32_t p,
                                 void *const *d_grad_ptrs, int32_t dtype,
                                 int32_t avg_mode, const int64_t *tokens,
                                 hipStream_t stream, ddp_comm_stats *stats);

/* ----------------------------------------------------------------------- */
/* Reducer: bucket all-reduces launched as gradients become ready           */
/* ----------------------------------------------------------------------- */

/* The reducer's bookkeeping ([DDP] Part 2 "Step 2: backward", items 2-3,
 * and "Step 3: finalize_backward"; [DP] "Overlapping communication with the
 * backward pass"). Each bucket has a pending count equal to its number of
 * parameters. ddp_reducer_mark_ready(param, ev) decrements the count of the
 * parameter's bucket; when a count reaches zero and that bucket is the next
 * to reduce, the reducer makes `comm_stream` wait for the events given with
 * the parameters of that bucket and of every following bucket that is also
 * complete, then launches that run of buckets with ddp_allreduce_buckets on
 * `comm_stream`. Buckets thus start in index order, each as soon as its
 * gradients and its predecessors allow, overlapping the producers' work.
 *
 *   create    plan (with ddp_plan_upload_segments done for p), p, the DEVICE
 *             gradient pointer table, dtype, averaging (tokens copied), and
 *             the stream the all-reduces run on. Plan and table must outlive
 *             the reducer. Errors: DDP_EINVAL, DDP_ERANGE; DDP_ENOTREADY
 *             when the plan's descriptor table was not uploaded for this p.
 *   prepare   starts a backward pass (all counts reset).
 *   mark_ready  param in [0, n_params); `ready` is an event recorded after
 *             that parameter's gradients of all ranks were written (NULL if
 *             they already were when the call is made). DDP_EINVAL for a
 *             second mark of a parameter in one pass or a mark outside a
 *             pass, DDP_ERANGE for a bad index. A failed launch returns its
 *             error, and every later mark_ready and the finalize of that
 *             pass return the same status with the same detail, until the
 *             next prepare.
 *   finalize  ends the pass. DDP_ENOTREADY (with the bucket and counts in
 *             ddp_last_error) if some bucket never became ready -- what DDP
 *             would wait for forever without find_unused_parameters.
 *             Otherwise `wait_stream` is made to wait for the all-reduces.
 *   launch_log  the runs launched in the current or last pass: the mark (0-
 *             based, in call order) that launched each run, its first bucket
 *             and its length; returns the number of runs (writes at most
 *             `capacity`).
 * Not thread-safe: one host thread drives a reducer. */
typedef struct ddp_reducer ddp_reducer;
ddp_status ddp_reducer_create(const ddp_plan *plan, int32_t p,
                              void *const *d_grad_ptrs, int32_t dtype,
                              int32_t avg_mode, const int64_t *tokens,
                              hipStream_t comm_stream, ddp_reducer **out);
void ddp_reducer_free(ddp_reducer *reducer);
ddp_status ddp_reducer_prepare(ddp_reducer *reducer);
ddp_status ddp_reducer_mark_ready(ddp_reducer *reducer, int32_t param,
                                  hipEvent_t ready);
ddp_status ddp_reducer_finalize(ddp_reducer *reducer, hipStream_t wait_stream);
int32_t ddp_reducer_launch_log(const ddp_reducer *reducer, int32_t *at_mark,
                               int32_t *first_bucket, int32_t *n_buckets,
                               int32_t capacity);
/* Cap the number of workgroups of every all-reduce launch the reducer makes
 * (0, the default: one workgroup per tile). On one device the bucket
 * all-reduces share the compute units with the kernels producing the
 * gradients; a capped launch walks its tiles with fewer workgroups and
 * leaves the rest of the GPU to the backward, as a collective library gives
 * a collective a fixed number of channels. Results are unchanged.
 * Errors: DDP_EINVAL for a NULL reducer or a negative cap. */
ddp_status ddp_reducer_set_max_workgroups(ddp_reducer *reducer,
                                          int32_t max_workgroups);
/* The parameters in the order they were marked ready in the current or last
 * pass (writes at most `capacity`; returns the count, -1 for NULL): the
 * order from which ddp_bucket_plan_ordered rebuilds the buckets. */
int32_t ddp_reducer_ready_order(const ddp_reducer *reducer, int32_t *order,
                                int32_t capacity);

/* ----------------------------------------------------------------------- */
/* Ring all-reduce                                                         */
/* ----------------------------------------------------------------------- */

/* In-place all-reduce of p rank buffers of n elements each ([COL] "Ring
 * allreduce in two passes"; [DP] "Ring all-reduce, derived"): zero-pad to a
 * multiple of p (the padding is never stored), p-1 reduce-scatter steps,
 * averaging by avg_mode, p-1 all-gather steps, trim. Afterwards every
 * rank's buffer holds the same bits.
 *
 *   bufs       HOST array of p device pointers (16-byte aligned, disjoint)
 *   n          elements per rank (>= 0; 0 is a no-op)
 *   dtype      DDP_F32 or DDP_BF16
 *   avg_mode   ddp_avg_mode; tokens is a HOST array of p counts (>= 0,
 *              sum > 0) read only for DDP_AVG_TOKENS
 *   algo       DDP_ALGO_FUSED or DDP_ALGO_RING
 *   workspace  device memory for DDP_ALGO_RING with bf16 (fp32 partials),
 *              ring_allreduce_sim_workspace() bytes, 16-byte aligned,
 *              disjoint from bufs; otherwise may be NULL
 *   stats      optional (NULL): filled with the schedule's accounting
 * Errors: DDP_EINVAL, DDP_ERANGE (p), DDP_EALIGN, DDP_EALIAS,
 * DDP_EWORKSPACE, DDP_EHIP (launch failure). */
ddp_status ring_allreduce_sim(void *const *bufs, int32_t p, int64_t n,
                              int32_t dtype, int32_t avg_mode,
                              const int64_t *tokens, int32_t algo,
                              void *workspace, size_t workspace_bytes,
                              hipStream_t stream, ddp_comm_stats *stats);

/* Workspace bytes ring_allreduce_sim needs (0 unless RING with bf16). */
size_t ring_allreduce_sim_workspace(int32_t p, int64_t n, int32_t dtype,
                                    int32_t algo);

/* For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc. The same
 * all-reduce as ring_allreduce_sim (same kernels, same bits), with the
 * workspace of DDP_ALGO_RING on bf16 taken from a scratch array of
 * DDP_NOALLOC_SCRATCH_BYTES that the library holds in device memory, one
 * per GPU, for the life of the process. Calls whose workspace would exceed
 * it (ring_allreduce_sim_workspace(p, n, dtype, algo) bytes) fail with
 * DDP_EWORKSPACE before anything is enqueued; the fused algorithm and fp32
 * need no workspace and have no limit. The call allocates nothing and
 * frees nothing. The array is overwritten before it is read, so what an
 * earlier call left there does not matter; but every call on one GPU uses
 * that GPU's single array, so calls whose bf16 rings can overlap in time on
 * one GPU (other streams, other host threads) race and must be ordered by
 * the caller. Errors: as ring_allreduce_sim, and DDP_EHIP if the array's
 * device address cannot be obtained. */
#define DDP_NOALLOC_SCRATCH_BYTES (64ll << 20)
ddp_status ring_allreduce_sim_noalloc(void *const *bufs, int32_t p, int64_t n,
                                      int32_t dtype, int32_t avg_mode,
                                      const int64_t *tokens, int32_t algo,
                                      hipStream_t stream, ddp_comm_stats *stats);

/* Run only ring steps [first_step, first_step + n_steps) of the 2(p-1)
 * steps of the fp32 ring schedule, in place: steps 0..p-2 are the
 * reduce-scatter steps (step p-2 also applies the averaging to each
 * owner's finished chunk), steps p-1..2p-3 the all-gather steps. Running
 * all steps in order equals ring_allreduce_sim with DDP_ALGO_RING. For
 * checking the schedule's intermediate states: after steps 0..k, rank
 * (j+k+1) mod p holds the partial sum of chunk j over ranks j..j+k+1.
 * Requires p >= 2 and dtype fp32 (buffers are float*).
 * Errors: as ring_allreduce_sim, plus DDP_ERANGE for the step range. */
ddp_status ring_allreduce_sim_steps(void *const *bufs, int32_t p, int64_t n,
                                    int32_t avg_mode, const int64_t *tokens,
                                    int32_t first_step, int32_t n_steps,
                                    hipStream_t stream);

/* ----------------------------------------------------------------------- */
/* All-reduce schedules and their choice by message size                   */
/* ----------------------------------------------------------------------- */

/* The all-reduce schedules ([DP] "Latency, trees, and choosing an
 * algorithm"; [COL], its exercise of a tree all-reduce beside the ring):
 *   DDP_SCHED_RING                the ring of ring_allreduce_sim.
 *   DDP_SCHED_RECURSIVE_DOUBLING  log2 p steps; in step j every rank swaps
 *                                 its whole buffer with rank r XOR 2^j and
 *                                 both add.
 *   DDP_SCHED_RABENSEIFNER        recursive halving (partner at distance
 *                                 p/2, then p/4, ...; each keeps the half
 *                                 of its range matching its own rank and
 *                                 adds the partner's copy of it), then
 *                                 recursive doubling of the owned ranges.
 *   DDP_SCHED_TREE                reduce up the doubling tree of
 *                                 broadcast_sim to rank 0, then broadcast
 *                                 down it; 2 ceil(log2 p) steps.
 * For p not a power of two (q = the largest power of two below p),
 * recursive doubling and Rabenseifner first fold each extra rank r >= q into
 * rank r - q and finally copy the result back to it. Each schedule fixes
 * its own summation order: the ring folds chunk c from rank c; recursive
 * doubling is a pairwise sum over ranks, nearest neighbours first;
 * Rabenseifner and the tree are the pairwise sum that pairs ranks q/2
 * apart first. Results differ between schedules in the last bits; each is
 * bit-identical to its literal schedule. */
typedef enum {
  DDP_SCHED_RING = 0,
  DDP_SCHED_RECURSIVE_DOUBLING = 1,
  DDP_SCHED_RABENSEIFNER = 2,
  DDP_SCHED_TREE = 3
} ddp_schedule;

/* In-place all-reduce of p rank buffers under `schedule`. Arguments as for
 * ring_allreduce_sim, except:
 *   schedule   ddp_schedule
 *   steps      0: one fused pass that reads each buffer once, folds every
 *              element in the schedule's order and writes all ranks
 *              (device traffic 2 p n bytes-per-element); 1: the schedule
 *              step by step, one kernel launch per step, each step moving
 *              the data its messages carry between rank buffers in device
 *              memory (bf16 runs on an fp32 workspace). Same bits either way.
 *   workspace  allreduce_sim_workspace() bytes (0 unless steps with bf16).
 * The stats describe the logical schedule (steps, messages, bytes per
 * rank on an fp32 wire) and the device traffic of the form that ran.
 * DDP_SCHED_RING is ring_allreduce_sim (steps selects DDP_ALGO_RING).
 * Errors: as ring_allreduce_sim; DDP_EINVAL for an unknown schedule. */
ddp_status allreduce_sim(void *const *bufs, int32_t p, int64_t n,
                         int32_t dtype, int32_t avg_mode,
                         const int64_t *tokens, int32_t schedule,
                         int32_t steps, void *workspace,
                         size_t workspace_bytes, hipStream_t stream,
                         ddp_comm_stats *stats);

/* Workspace bytes allreduce_sim needs (0 unless steps == 1 with bf16). */
size_t allreduce_sim_workspace(int32_t p, int64_t n, int32_t dtype,
                               int32_t schedule, int32_t steps);

/* Latency-bandwidth (Hockney) time of one all-reduce of `bytes` under a
 * schedule ([DP] "Ring all-reduce, derived" and "Latency, trees, and
 * choosing an algorithm"): alpha seconds per step plus beta seconds per
 * byte of each step's largest message. For p a power of two: ring
 * 2(p-1)(alpha + beta bytes/p); recursive doubling
 * log2 p (alpha + beta bytes); Rabenseifner 2 log2 p alpha +
 * 2(p-1)/p bytes beta; tree 2 log2 p (alpha + beta bytes). Other p add the
 * two whole-buffer steps of the extra ranks (the tree takes
 * 2 ceil(log2 p) steps). Returns a negative value for bad arguments. */
double ddp_schedule_time(int32_t schedule, int32_t p, double bytes,
                         double alpha, double beta);

/* The schedule with the smallest ddp_schedule_time among the candidates
 * (bit s of `candidates` set = schedule s allowed), ties to the lower
 * schedule number: libraries pick the algorithm per call from the message
 * size ([DP] "Latency, trees, and choosing an algorithm"; [COL] describes
 * NCCL taking the ring for large messages and a tree for small ones).
 * With the ring and recursive doubling as candidates the choice flips at
 * the crossover size the page derives.
 * Returns -1 (with ddp_last_error) for bad arguments or no candidate. */
int32_t ddp_choose_schedule(int32_t p, int64_t bytes, double alpha,
                            double beta, uint32_t candidates);

/* Step time of a backward pass whose bucket all-reduces overlap it ([DP]
 * "Overlapping communication with the backward pass": the step-time
 * exercise there, whose printed stub has no overlap at all, taken with the
 * overlap the section describes). Bucket b's all-reduce starts once the last
 * of its parameters is ready and bucket b-1's all-reduce has finished
 * (buckets run one at a time in index order, as the reducer launches them)
 * and lasts bucket_time[b]. The backward ends at the latest ready time; the
 * step ends when the backward and the last all-reduce have both finished;
 * the exposed time is step minus the end of backward.
 *   plan         bucket plan: the parameters of each bucket
 *   ready        HOST array of ddp_plan_num_params(plan) times, in seconds
 *                from the start of backward, at which each parameter's
 *                gradient is ready (registration index order)
 *   bucket_time  HOST array of ddp_plan_num_buckets(plan) all-reduce
 *                durations in seconds: ddp_schedule_time of each bucket's
 *                bytes for a network, or kernel times measured on a device
 *   step, exposed  outputs (either may be NULL)
 * Every time must be finite and >= 0; an array may be NULL when the plan
 * has no parameters. Errors: DDP_EINVAL (NULL plan, a NULL array the plan
 * needs, a negative, NaN or infinite time); outputs untouched then. */
ddp_status ddp_overlap_step_time(const ddp_plan *plan, const double *ready,
                                 const double *bucket_time, double *step,
                                 double *exposed);

/* ----------------------------------------------------------------------- */
/* Standalone collectives                                                  */
/* ----------------------------------------------------------------------- */

/* Reduce-scatter ([COL], the implementation's reduce_scatter: the first ring
 * pass pre-rotated so rank r ends with chunk r; [DP] "The collective
 * operations"): out[r][i] = avg(sum over ranks of in[.][r*C + i]),
 * C = n/p, folded in ring order starting at rank (r+1) mod p.
 *   in   HOST array of p device pointers to n elements (read only)
 *   out  HOST array of p device pointers to C elements (element-aligned;
 *        16-byte alignment and C a whole number of 16-byte vectors take the
 *        vector path); out[r] may equal
 *        in[r] + r*C elements (in place), otherwise it must not overlap any
 *        input or output
 * Errors: DDP_ENOTDIVISIBLE when n % p != 0, plus those of
 * ring_allreduce_sim. */
ddp_status reduce_scatter_sim(const void *const *in, void *const *out,
                              int32_t p, int64_t n, int32_t dtype,
                              int32_t avg_mode, const int64_t *tokens,
                              hipStream_t stream, ddp_comm_stats *stats);

/* All-gather ([COL], allgather by ring rotations; [DP] "The collective
 * operations"): out[r] = in[0] || in[1] || ... || in[p-1] for every r.
 *   n    elements of each OUTPUT buffer (n % p == 0); shards hold n/p
 *   in   HOST array of p device pointers to n/p elements; in[r] may equal
 *        out[r] + r*(n/p) elements (in place: that slice is then not
 *        rewritten), otherwise inputs must not overlap any output
 *   out  HOST array of p device pointers to n elements, disjoint
 * dtype only sets the element size. */
ddp_status allgather_sim(const void *const *in, void *const *out, int32_t p,
                         int64_t n, int32_t dtype, hipStream_t stream,
                         ddp_comm_stats *stats);

/* Broadcast ([COL], broadcast over a doubling tree): every rank's buffer
 * receives a copy of bufs[src]'s n elements, in place. The stats describe
 * the doubling tree (ceil(log2 p) rounds, p-1 messages); on one device the
 * copy is one pass that reads the source once. */
ddp_status broadcast_sim(void *const *bufs, int32_t p, int64_t n,
                         int32_t src, int32_t dtype, hipStream_t stream,
                         ddp_comm_stats *stats);

/* Broadcast of many tensors from rank `root`, coalesced into the buckets of
 * a plan from ddp_coalesce_plan (or any uploaded plan): afterwards every
 * rank's copy of every tensor holds the root's bytes. This is DDP's
 * init-time synchronisation of parameters and buffers (root 0; [DDP] Part 1,
 * "_sync_module_states") and its per-forward buffer broadcast from the
 * authoritative rank ([DDP] Part 2, "_pre_forward" and the chain to the
 * coalesced broadcast). One launch per bucket, in bucket order, reads the
 * root's tensors once and writes the other p - 1 copies (no staging buffer;
 * device traffic p bytes-per-element). The stats describe the pages' form:
 * per bucket one flat message down the doubling tree (ceil(log2 p) rounds,
 * p - 1 messages of the bucket's bytes).
 *   d_tensor_ptrs  DEVICE array of p * n_tensors addresses, rank-major
 *                  (rank r's copy of tensor i at r * n_tensors + i), each
 *                  aligned to the element size; copies of different ranks
 *                  or tensors must not overlap (not checked)
 * Errors: DDP_ENOTREADY (plan not uploaded), DDP_ERANGE (p, root),
 * DDP_EINVAL. */
ddp_status ddp_broadcast_coalesced(const ddp_plan *plan, int32_t p,
                                   void *const *d_tensor_ptrs, int32_t root,
                                   hipStream_t stream, ddp_comm_stats *stats);


#ifdef __cplusplus
}
#endif

#endif /* DDPSIM_H */
