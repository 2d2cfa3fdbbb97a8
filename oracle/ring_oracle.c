/*
 * ring_oracle.c -- plain, single-threaded CPU oracle for the bucketed
 * data-parallel gradient-synchronisation path.
 *
 * TEST INFRASTRUCTURE ONLY. The test suite, the smoke check and the
 * benchmark's CPU-baseline leg are the only callers. The HIP library never
 * links, loads or calls this file, and the two share no source, header,
 * table or helper.
 *
 * Build (see oracle/__init__.py):
 *   gcc -O2 -std=c11 -fno-fast-math -ffp-contract=off -fPIC -shared
 * so every fp32 operation below is one IEEE-754 binary32 operation with
 * round-to-nearest-even: no FMA contraction, no reassociation, no flush of
 * subnormals, division correctly rounded.
 *
 * Sources, cited by page title and section:
 *   [DDP] "PyTorch DDP Deep Dive -- Initialization, Buffer Broadcast, the
 *         Reducer, and the torch.compile Story"
 *   [COL] "Collective Ops From Scratch"
 *   [DP]  "Data parallelism" (zerotofrontier.app, distributed chapter)
 *
 * What is computed, and where it comes from:
 *   orc_bucket_plan     reverse-registration greedy bucketing with a small
 *                       first bucket ([DDP] Part 1 "What _ddp_init_helper
 *                       actually does"; [DDP] Part 3, the DDPOptimizer
 *                       reverse walk; [DP] "Overlapping communication with
 *                       the backward pass").
 *   orc_flatten /       copy each parameter's gradient into / out of its slot
 *   orc_unflatten       of the bucket's flat buffer, optional pre-divide
 *                       ([DDP] Part 2 "Step 2: backward", item 1, and
 *                       "Step 3: finalize_backward").
 *   orc_ring_allreduce  zero-pad to a multiple of p, p-1 reduce-scatter steps,
 *                       p-1 all-gather steps, trim ([COL] "Ring allreduce in
 *                       two passes"; [DP] "Ring all-reduce, derived"), with
 *                       explicit send buffers and a message log.
 *   orc_reduce_scatter  the first pass alone, pre-rotated so rank r ends with
 *                       chunk r; n must divide by p ([COL] list of what the
 *                       implementation provides).
 *   orc_allgather       p-1 ring rotations of shards ([COL]; [DP] "The
 *                       collective operations").
 *   orc_broadcast       doubling (binomial) tree from src ([COL]).
 *   orc_fold_samples    the per-element value the ring reaches, written as a
 *                       fold over ranks (derived from the chunk's journey in
 *                       [DP] "Ring all-reduce, derived"); pinned in tests to
 *                       the literal simulation.
 *   orc_allreduce       the all-reduce under a chosen schedule: the ring, or
 *                       one of the logarithmic-latency schedules of [DP]
 *                       "Latency, trees, and choosing an algorithm"
 *                       (recursive doubling; recursive halving then doubling,
 *                       i.e. Rabenseifner's algorithm) or the tree all-reduce
 *                       that [COL] sets as an exercise (reduce up the
 *                       doubling tree, broadcast down it).
 *   orc_bucket_plan_ordered  the bucketing rule over an explicit order (the
 *                       rebuild from the observed ready order, [DDP] Part 2).
 *   orc_broadcast_coalesced  many tensors broadcast in capped buckets:
 *                       flatten at the root, doubling-tree broadcast,
 *                       unflatten everywhere ([DDP] Parts 1 and 2).
 *   orc_tree_fold_samples  the per-element value those schedules reach,
 *                       written as a pairwise fold; pinned to the literal
 *                       simulations in tests.
 *
 * Readings where the pages leave a step open (also listed in the design
 * notes): equal chunks of ceil(n/p) with the padding at the end; averaging is
 * one correctly rounded fp32 division of the finished sum by (float)p or by
 * (float)(total tokens); bf16 inputs are widened exactly, folded in fp32 and
 * rounded once to bf16 with round-to-nearest-even; the "wire" of a bf16 ring
 * carries fp32 partials.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_OK 0
#define ORC_EINVAL (-1)
#define ORC_ENOTDIVISIBLE (-2)
#define ORC_ENOMEM (-3)

#define ORC_AVG_NONE 0
#define ORC_AVG_WORLD 1
#define ORC_AVG_TOKENS 2

#define ORC_PHASE_REDUCE_SCATTER 0
#define ORC_PHASE_ALLGATHER 1
#define ORC_PHASE_BROADCAST 2
#define ORC_PHASE_EXCHANGE 3  /* recursive doubling: whole buffers swapped  */
#define ORC_PHASE_FOLD_IN 4   /* p not a power of two: extra rank -> core   */
#define ORC_PHASE_FOLD_OUT 5  /* ... and the result back to the extra rank  */
#define ORC_PHASE_REDUCE 6    /* tree all-reduce: towards rank 0            */

#define ORC_SCHED_RING 0
#define ORC_SCHED_RECURSIVE_DOUBLING 1
#define ORC_SCHED_RABENSEIFNER 2
#define ORC_SCHED_TREE 3

/* One logged message: who sent which chunk to whom, in which step. */
typedef struct {
  int32_t phase;
  int32_t step;
  int32_t src;
  int32_t dst;
  int32_t chunk;
  int32_t reserved;
  int64_t bytes;
} orc_msg;

typedef struct {
  orc_msg *entries;
  int64_t capacity;
  int64_t count;
} msg_log;

static void log_msg(msg_log *log, int32_t phase, int32_t step, int32_t src,
                    int32_t dst, int32_t chunk, int64_t bytes) {
  if (log->entries != NULL && log->count < log->capacity) {
    orc_msg *m = &log->entries[log->count];
    m->phase = phase;
    m->step = step;
    m->src = src;
    m->dst = dst;
    m->chunk = chunk;
    m->reserved = 0;
    m->bytes = bytes;
  }
  log->count += 1;
}

static int32_t mod_p(int64_t a, int32_t p) {
  int64_t m = a % p;
  return (int32_t)(m < 0 ? m + p : m);
}

/* ------------------------------------------------------------------------ */
/* bf16 <-> fp32                                                             */
/* ------------------------------------------------------------------------ */

/* bf16 is the upper half of a binary32, so widening is exact. */
float orc_bf16_to_f32(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return f;
}

/* Round a binary32 to the nearest bf16, ties to the even neighbour.
 * Written from the definition: keep the upper 16 bits, then look at the 16
 * discarded bits. Above half way rounds up, below rounds down, exactly half
 * way rounds to whichever neighbour has a zero last bit. A carry out of the
 * mantissa moves into the exponent, which is the correct next value
 * (including overflow to infinity). NaN stays a quiet NaN. */
uint16_t orc_f32_to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  uint32_t upper = u >> 16;
  uint32_t lower = u & 0xFFFFu;
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu) != 0) {
    return (uint16_t)(upper | 0x0040u);
  }
  if (lower > 0x8000u || (lower == 0x8000u && (upper & 1u))) {
    upper += 1;
  }
  return (uint16_t)upper;
}

void orc_f32_to_bf16_array(const float *in, uint16_t *out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_f32_to_bf16(in[i]);
}

void orc_bf16_to_f32_array(const uint16_t *in, float *out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_bf16_to_f32(in[i]);
}

/* ------------------------------------------------------------------------ */
/* Averaging divisor                                                         */
/* ------------------------------------------------------------------------ */

/* World averaging divides by the number of ranks ([DP] "Overlapping
 * communication with the backward pass", last paragraph). Token averaging
 * sums per-rank token counts across all ranks and divides the summed
 * gradient once by that total ([DP] "Why averaging gradients is exactly
 * large-batch training"). The divisor is the binary32 nearest the integer. */
static int avg_divisor(int32_t mode, int32_t p, const int64_t *tokens,
                       float *divisor) {
  if (mode == ORC_AVG_NONE) {
    *divisor = 1.0f;
    return ORC_OK;
  }
  if (mode == ORC_AVG_WORLD) {
    *divisor = (float)p;
    return ORC_OK;
  }
  if (mode == ORC_AVG_TOKENS) {
    if (tokens == NULL) return ORC_EINVAL;
    int64_t total = 0;
    for (int32_t r = 0; r < p; ++r) {
      if (tokens[r] < 0) return ORC_EINVAL;
      total += tokens[r];
    }
    if (total <= 0) return ORC_EINVAL;
    *divisor = (float)total;
    return ORC_OK;
  }
  return ORC_EINVAL;
}

int orc_avg_divisor(int32_t mode, int32_t p, const int64_t *tokens,
                    float *divisor) {
  if (p < 1) return ORC_EINVAL;
  return avg_divisor(mode, p, tokens, divisor);
}

/* ------------------------------------------------------------------------ */
/* Bucket plan                                                               */
/* ------------------------------------------------------------------------ */

/* Walk the parameters from the last registered to the first (the order in
 * which backward produces their gradients). Before adding a parameter, if
 * the open bucket holds at least one parameter and its byte size has reached
 * its cap, close it and open a new one. The cap of the first bucket filled
 * is min(first_cap, cap); every later bucket's cap is `cap`. A bucket can
 * therefore overshoot its cap by its last parameter, and no bucket is empty.
 *
 * Outputs:
 *   fill_order[k]     k-th parameter in fill order (bucket 0 first)
 *   bucket_begin[b]   index into fill_order where bucket b starts;
 *                     bucket_begin[n_buckets] == n_params
 *   offset[i]         element offset of parameter i inside its bucket
 *   bucket_of[i]      bucket that holds parameter i
 */
/* The same greedy bucketing over an explicit walk order: walk[k] is the
 * k-th parameter to place (a permutation of 0..n_params-1), or NULL for the
 * reverse registration order above. DDP rebuilds its buckets once from the
 * order in which gradients actually became ready in the first backward pass
 * ("PyTorch DDP Deep Dive", Part 2: the hook records each ready parameter
 * while buckets are due for a rebuild, and the rebuild runs before the next
 * forward); the rule applied to that order is the same. */
int orc_bucket_plan_ordered(const int64_t *numel, int32_t n_params,
                            const int32_t *walk, int32_t elem_bytes,
                            int64_t cap, int64_t first_cap,
                            int32_t *fill_order, int32_t *bucket_begin,
                            int64_t *offset, int32_t *bucket_of,
                            int32_t *n_buckets) {
  if (n_params < 0 || elem_bytes <= 0 || cap < 0 || first_cap < 0) {
    return ORC_EINVAL;
  }
  for (int32_t i = 0; i < n_params; ++i) {
    if (numel[i] < 0) return ORC_EINVAL;
  }
  if (walk != NULL) {
    char *seen = (char *)calloc((size_t)n_params + 1, 1);
    if (seen == NULL) return ORC_ENOMEM;
    int bad = 0;
    for (int32_t k = 0; k < n_params && !bad; ++k) {
      if (walk[k] < 0 || walk[k] >= n_params || seen[walk[k]]) bad = 1;
      else seen[walk[k]] = 1;
    }
    free(seen);
    if (bad) return ORC_EINVAL;
  }
  int32_t buckets = 0;       /* buckets opened so far */
  int32_t filled = 0;        /* parameters placed so far */
  int64_t open_elems = 0;    /* elements in the open bucket */
  int32_t open_count = 0;    /* parameters in the open bucket */
  for (int32_t k = 0; k < n_params; ++k) {
    int32_t i = walk != NULL ? walk[k] : n_params - 1 - k;
    if (buckets == 0) {
      buckets = 1;
      bucket_begin[0] = 0;
    } else {
      int64_t limit = cap;
      if (buckets == 1 && first_cap < cap) limit = first_cap;
      if (open_count > 0 && open_elems * elem_bytes >= limit) {
        bucket_begin[buckets] = filled;
        buckets += 1;
        open_elems = 0;
        open_count = 0;
      }
    }
    fill_order[filled] = i;
    offset[i] = open_elems;
    bucket_of[i] = buckets - 1;
    open_elems += numel[i];
    open_count += 1;
    filled += 1;
  }
  bucket_begin[buckets] = filled;
  *n_buckets = buckets;
  return ORC_OK;
}

int orc_bucket_plan(const int64_t *numel, int32_t n_params, int32_t elem_bytes,
                    int64_t cap, int64_t first_cap, int32_t *fill_order,
                    int32_t *bucket_begin, int64_t *offset, int32_t *bucket_of,
                    int32_t *n_buckets) {
  return orc_bucket_plan_ordered(numel, n_params, NULL, elem_bytes, cap,
                                 first_cap, fill_order, bucket_begin, offset,
                                 bucket_of, n_buckets);
}

/* Coalescing for a broadcast of many tensors ("PyTorch DDP Deep Dive", Part
 * 2, the buffer broadcast and the chain down to the coalesced broadcast,
 * whose buckets are capped at 250 MiB): tensors are taken in list order and
 * a bucket is closed before a tensor that would take it past the cap, so no
 * bucket exceeds the cap unless one tensor alone does. (The pages give only
 * the cap; "never past it" is the reading taken.) Outputs as for
 * orc_bucket_plan; fill order is list order. */
int orc_coalesce_plan(const int64_t *numel, int32_t n, int32_t elem_bytes,
                      int64_t cap, int32_t *fill_order, int32_t *bucket_begin,
                      int64_t *offset, int32_t *bucket_of, int32_t *n_buckets) {
  if (n < 0 || elem_bytes <= 0 || cap < 0) return ORC_EINVAL;
  for (int32_t i = 0; i < n; ++i) {
    if (numel[i] < 0) return ORC_EINVAL;
  }
  int32_t buckets = 0;
  int64_t open_elems = 0;
  int32_t open_count = 0;
  for (int32_t i = 0; i < n; ++i) {
    if (buckets == 0) {
      buckets = 1;
      bucket_begin[0] = 0;
    } else if (open_count > 0 && (open_elems + numel[i]) * elem_bytes > cap) {
      bucket_begin[buckets] = i;
      buckets += 1;
      open_elems = 0;
      open_count = 0;
    }
    fill_order[i] = i;
    offset[i] = open_elems;
    bucket_of[i] = buckets - 1;
    open_elems += numel[i];
    open_count += 1;
  }
  bucket_begin[buckets] = n;
  *n_buckets = buckets;
  return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Flatten / unflatten (one rank)                                            */
/* ------------------------------------------------------------------------ */

/* Copy every gradient of bucket `b` into the flat buffer at its offset. With
 * divisor != 1 each element is divided on the way in, as the reducer does
 * when it pre-divides by the world size. dtype 0 = fp32, 1 = bf16 (the
 * division then happens in fp32 and rounds once to bf16). */
int orc_flatten(const void *const *grads, const int64_t *numel,
                const int32_t *fill_order, const int32_t *bucket_begin,
                const int64_t *offset, int32_t b, int32_t dtype, float divisor,
                void *flat) {
  if (dtype != 0 && dtype != 1) return ORC_EINVAL;
  for (int32_t k = bucket_begin[b]; k < bucket_begin[b + 1]; ++k) {
    int32_t i = fill_order[k];
    int64_t n = numel[i];
    if (dtype == 0) {
      const float *g = (const float *)grads[i];
      float *dst = (float *)flat + offset[i];
      for (int64_t j = 0; j < n; ++j) {
        dst[j] = (divisor == 1.0f) ? g[j] : g[j] / divisor;
      }
    } else {
      const uint16_t *g = (const uint16_t *)grads[i];
      uint16_t *dst = (uint16_t *)flat + offset[i];
      for (int64_t j = 0; j < n; ++j) {
        dst[j] = (divisor == 1.0f)
                     ? g[j]
                     : orc_f32_to_bf16(orc_bf16_to_f32(g[j]) / divisor);
      }
    }
  }
  return ORC_OK;
}

/* Copy each slice of the reduced flat buffer back to its gradient. */
int orc_unflatten(void *const *grads, const int64_t *numel,
                  const int32_t *fill_order, const int32_t *bucket_begin,
                  const int64_t *offset, int32_t b, int32_t elem_bytes,
                  const void *flat) {
  if (elem_bytes <= 0) return ORC_EINVAL;
  for (int32_t k = bucket_begin[b]; k < bucket_begin[b + 1]; ++k) {
    int32_t i = fill_order[k];
    memcpy(grads[i], (const char *)flat + offset[i] * elem_bytes,
           (size_t)(numel[i] * elem_bytes));
  }
  return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* The literal ring, on p padded fp32 arrays                                 */
/* ------------------------------------------------------------------------ */

/* work[r] holds rank r's padded array of p*C floats. Runs at most
 * `max_steps` of the 2(p-1) ring steps (a negative value runs all of them).
 * Every step first copies each rank's outgoing chunk into its own send
 * buffer, then delivers all messages, so within a step no rank reads a value
 * another rank wrote in that same step.
 *
 * Reduce-scatter step k (k = 0..p-2): rank r sends chunk (r - k - shift) mod p
 * to rank r+1, which adds it into its own copy. With shift = 0 this is the
 * all-reduce schedule ([COL] "Ring allreduce in two passes"; [DP] "Ring
 * all-reduce, derived", phase 1) and leaves rank q owning chunk (q+1) mod p.
 * shift = 1 is the pre-rotated standalone reduce-scatter, leaving rank q
 * owning chunk q.
 *
 * When the reduce-scatter phase is complete, each owner divides its finished
 * chunk by the divisor (if averaging), so the all-gather hands out averages.
 *
 * All-gather step k: rank r sends chunk (r + 1 - k) mod p to rank r+1, which
 * overwrites its copy ([DP] "Ring all-reduce, derived", phase 2).
 *
 * Returns the number of steps executed. */
static int32_t ring_on_work(float **work, float **send, int32_t p, int64_t C,
                            int32_t shift, int32_t run_allgather,
                            int32_t max_steps, int32_t do_divide,
                            float divisor, int64_t wire_bytes, msg_log *log) {
  int32_t done = 0;
  for (int32_t k = 0; k <= p - 2; ++k) {
    if (max_steps >= 0 && done >= max_steps) return done;
    for (int32_t r = 0; r < p; ++r) {
      int32_t j = mod_p((int64_t)r - k - shift, p);
      memcpy(send[r], work[r] + (int64_t)j * C, (size_t)C * sizeof(float));
      log_msg(log, ORC_PHASE_REDUCE_SCATTER, k, r, (r + 1) % p, j,
              C * wire_bytes);
    }
    for (int32_t r = 0; r < p; ++r) {
      int32_t dst = (r + 1) % p;
      int32_t j = mod_p((int64_t)r - k - shift, p);
      float *mine = work[dst] + (int64_t)j * C;
      for (int64_t e = 0; e < C; ++e) mine[e] = mine[e] + send[r][e];
    }
    done += 1;
  }
  if (do_divide) {
    for (int32_t q = 0; q < p; ++q) {
      int32_t j = mod_p((int64_t)q + 1 - shift, p);
      float *mine = work[q] + (int64_t)j * C;
      for (int64_t e = 0; e < C; ++e) mine[e] = mine[e] / divisor;
    }
  }
  if (!run_allgather) return done;
  for (int32_t k = 0; k <= p - 2; ++k) {
    if (max_steps >= 0 && done >= max_steps) return done;
    for (int32_t r = 0; r < p; ++r) {
      int32_t j = mod_p((int64_t)r + 1 - k, p);
      memcpy(send[r], work[r] + (int64_t)j * C, (size_t)C * sizeof(float));
      log_msg(log, ORC_PHASE_ALLGATHER, k, r, (r + 1) % p, j, C * wire_bytes);
    }
    for (int32_t r = 0; r < p; ++r) {
      int32_t dst = (r + 1) % p;
      int32_t j = mod_p((int64_t)r + 1 - k, p);
      memcpy(work[dst] + (int64_t)j * C, send[r], (size_t)C * sizeof(float));
    }
    done += 1;
  }
  return done;
}

static void free_arrays(float **a, int32_t p) {
  if (a == NULL) return;
  for (int32_t r = 0; r < p; ++r) free(a[r]);
  free(a);
}

static float **alloc_arrays(int32_t p, int64_t len) {
  float **a = (float **)calloc((size_t)p, sizeof(float *));
  if (a == NULL) return NULL;
  for (int32_t r = 0; r < p; ++r) {
    /* calloc: the padding elements start at +0.0 */
    a[r] = (float *)calloc((size_t)(len > 0 ? len : 1), sizeof(float));
    if (a[r] == NULL) {
      free_arrays(a, p);
      return NULL;
    }
  }
  return a;
}

/* Ring all-reduce of p rank arrays of n elements, in place.
 * dtype 0: bufs are float*; dtype 1: bufs are bf16 (uint16_t*).
 * avg_mode: ORC_AVG_NONE / ORC_AVG_WORLD / ORC_AVG_TOKENS (tokens[p]).
 * max_steps < 0 runs the whole schedule; otherwise only the first max_steps
 * ring steps run (the divide happens once the reduce-scatter phase is done)
 * and the partial state is written back, trimmed to n.
 * log/log_capacity may be NULL/0; *n_msgs receives the message count.
 * Padding: C = ceil(n/p) elements per chunk, zeros at the end, trimmed. */
int orc_ring_allreduce(void *const *bufs, int32_t p, int64_t n, int32_t dtype,
                       int32_t avg_mode, const int64_t *tokens,
                       int32_t max_steps, orc_msg *log, int64_t log_capacity,
                       int64_t *n_msgs) {
  if (p < 1 || n < 0 || (dtype != 0 && dtype != 1)) return ORC_EINVAL;
  float divisor = 1.0f;
  int rc = avg_divisor(avg_mode, p, tokens, &divisor);
  if (rc != ORC_OK) return rc;
  int64_t C = (n + p - 1) / p;
  int64_t n_pad = C * p;
  float **work = alloc_arrays(p, n_pad);
  float **send = alloc_arrays(p, C);
  if (work == NULL || send == NULL) {
    free_arrays(work, p);
    free_arrays(send, p);
    return ORC_ENOMEM;
  }
  for (int32_t r = 0; r < p; ++r) {
    if (dtype == 0) {
      memcpy(work[r], bufs[r], (size_t)n * sizeof(float));
    } else {
      orc_bf16_to_f32_array((const uint16_t *)bufs[r], work[r], n);
    }
  }
  msg_log lg = {log, log_capacity, 0};
  /* The wire carries fp32 values for both dtypes. */
  ring_on_work(work, send, p, C, /*shift=*/0, /*run_allgather=*/1, max_steps,
               avg_mode != ORC_AVG_NONE, divisor, (int64_t)sizeof(float), &lg);
  for (int32_t r = 0; r < p; ++r) {
    if (dtype == 0) {
      memcpy(bufs[r], work[r], (size_t)n * sizeof(float));
    } else {
      orc_f32_to_bf16_array(work[r], (uint16_t *)bufs[r], n);
    }
  }
  if (n_msgs != NULL) *n_msgs = lg.count;
  free_arrays(work, p);
  free_arrays(send, p);
  return ORC_OK;
}

/* Standalone reduce-scatter: in[r] has n elements (n divisible by p),
 * out[r] receives the (averaged) sum of chunk r, C = n/p elements. The
 * schedule is the ring's first pass with the chunk index shifted by one, so
 * rank r finishes owning chunk r. */
int orc_reduce_scatter(const void *const *in, void *const *out, int32_t p,
                       int64_t n, int32_t dtype, int32_t avg_mode,
                       const int64_t *tokens, orc_msg *log,
                       int64_t log_capacity, int64_t *n_msgs) {
  if (p < 1 || n < 0 || (dtype != 0 && dtype != 1)) return ORC_EINVAL;
  if (n % p != 0) return ORC_ENOTDIVISIBLE;
  float divisor = 1.0f;
  int rc = avg_divisor(avg_mode, p, tokens, &divisor);
  if (rc != ORC_OK) return rc;
  int64_t C = n / p;
  float **work = alloc_arrays(p, n);
  float **send = alloc_arrays(p, C);
  if (work == NULL || send == NULL) {
    free_arrays(work, p);
    free_arrays(send, p);
    return ORC_ENOMEM;
  }
  for (int32_t r = 0; r < p; ++r) {
    if (dtype == 0) {
      memcpy(work[r], in[r], (size_t)n * sizeof(float));
    } else {
      orc_bf16_to_f32_array((const uint16_t *)in[r], work[r], n);
    }
  }
  msg_log lg = {log, log_capacity, 0};
  ring_on_work(work, send, p, C, /*shift=*/1, /*run_allgather=*/0, -1,
               avg_mode != ORC_AVG_NONE, divisor, (int64_t)sizeof(float), &lg);
  for (int32_t r = 0; r < p; ++r) {
    const float *mine = work[r] + (int64_t)r * C;
    if (dtype == 0) {
      memcpy(out[r], mine, (size_t)C * sizeof(float));
    } else {
      orc_f32_to_bf16_array(mine, (uint16_t *)out[r], C);
    }
  }
  if (n_msgs != NULL) *n_msgs = lg.count;
  free_arrays(work, p);
  free_arrays(send, p);
  return ORC_OK;
}

/* Standalone all-gather: in[r] is rank r's shard of `shard` elements of
 * elem_bytes each; out[r] receives the rank-ordered concatenation of all
 * shards (p*shard elements). Schedule: p-1 ring rotations; at step k rank r
 * forwards the shard of rank (r - k) mod p to rank r+1. */
int orc_allgather(const void *const *in, void *const *out, int32_t p,
                  int64_t shard, int32_t elem_bytes, orc_msg *log,
                  int64_t log_capacity, int64_t *n_msgs) {
  if (p < 1 || shard < 0 || elem_bytes <= 0) return ORC_EINVAL;
  size_t sb = (size_t)(shard * elem_bytes);
  char **have = (char **)calloc((size_t)p, sizeof(char *));
  char **send = (char **)calloc((size_t)p, sizeof(char *));
  if (have == NULL || send == NULL) {
    free(have);
    free(send);
    return ORC_ENOMEM;
  }
  int fail = 0;
  for (int32_t r = 0; r < p && !fail; ++r) {
    have[r] = (char *)calloc((size_t)p * sb + 1, 1);
    send[r] = (char *)calloc(sb + 1, 1);
    if (have[r] == NULL || send[r] == NULL) fail = 1;
  }
  if (!fail) {
    msg_log lg = {log, log_capacity, 0};
    for (int32_t r = 0; r < p; ++r) {
      memcpy(have[r] + (size_t)r * sb, in[r], sb);
    }
    for (int32_t k = 0; k <= p - 2; ++k) {
      for (int32_t r = 0; r < p; ++r) {
        int32_t j = mod_p((int64_t)r - k, p);
        memcpy(send[r], have[r] + (size_t)j * sb, sb);
        log_msg(&lg, ORC_PHASE_ALLGATHER, k, r, (r + 1) % p, j, (int64_t)sb);
      }
      for (int32_t r = 0; r < p; ++r) {
        int32_t j = mod_p((int64_t)r - k, p);
        memcpy(have[(r + 1) % p] + (size_t)j * sb, send[r], sb);
      }
    }
    for (int32_t r = 0; r < p; ++r) memcpy(out[r], have[r], (size_t)p * sb);
    if (n_msgs != NULL) *n_msgs = lg.count;
  }
  for (int32_t r = 0; r < p; ++r) {
    free(have[r]);
    free(send[r]);
  }
  free(have);
  free(send);
  return fail ? ORC_ENOMEM : ORC_OK;
}

/* Broadcast over a doubling tree, in place: bufs[src] is copied to every
 * rank. With relative rank v = (r - src) mod p, in round j every rank with
 * v < 2^j that already holds the data sends it to v + 2^j (if that rank
 * exists). ceil(log2 p) rounds. */
int orc_broadcast(void *const *bufs, int32_t p, int64_t n, int32_t elem_bytes,
                  int32_t src, orc_msg *log, int64_t log_capacity,
                  int64_t *n_msgs) {
  if (p < 1 || n < 0 || elem_bytes <= 0 || src < 0 || src >= p) {
    return ORC_EINVAL;
  }
  size_t nb = (size_t)(n * elem_bytes);
  msg_log lg = {log, log_capacity, 0};
  int32_t round = 0;
  for (int64_t span = 1; span < p; span *= 2, ++round) {
    for (int64_t v = 0; v < span; ++v) {
      int64_t to = v + span;
      if (to >= p) continue;
      int32_t s = (int32_t)((v + src) % p);
      int32_t d = (int32_t)((to + src) % p);
      memcpy(bufs[d], bufs[s], nb);
      log_msg(&lg, ORC_PHASE_BROADCAST, round, s, d, 0, (int64_t)nb);
    }
  }
  if (n_msgs != NULL) *n_msgs = lg.count;
  return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* The ring's result at single elements                                      */
/* ------------------------------------------------------------------------ */

/* For each sample s: vals[s*p + r] is rank r's value at that element and
 * start[s] the rank whose contribution the ring takes first (the element's
 * chunk index for the all-reduce; chunk + 1 for the pre-rotated
 * reduce-scatter). Following one chunk around the ring, every hop adds the
 * next rank's untouched original value, so the finished sum is
 *   x[start] + x[start+1] + ... + x[start+p-1]   (indices mod p),
 * accumulated left to right in fp32, then divided once if averaging. */
void orc_fold_samples(const float *vals, const int64_t *start, int32_t p,
                      int64_t count, int32_t do_divide, float divisor,
                      float *out) {
  for (int64_t s = 0; s < count; ++s) {
    const float *x = vals + s * p;
    int32_t c = mod_p(start[s], p);
    float acc = x[c];
    for (int32_t t = 1; t < p; ++t) acc = acc + x[(c + t) % p];
    out[s] = do_divide ? acc / divisor : acc;
  }
}

/* ------------------------------------------------------------------------ */
/* Reducer schedule: when each bucket's all-reduce is launched             */
/* ------------------------------------------------------------------------ */

/* The reducer's readiness bookkeeping ("PyTorch DDP Deep Dive", Part 2
 * "Step 2: backward"): every bucket starts with a pending count equal to
 * its number of parameters. Marking a parameter ready decrements its
 * bucket's count; when a count reaches zero and that bucket is the next one
 * to reduce, the reducer launches it and keeps launching following buckets
 * while they are complete too. A bucket that completes out of turn waits.
 *
 * Inputs: bucket_of[n_params]; n_buckets; order[n_marks] = parameters in the
 * order they are marked ready.
 * Outputs, per mark m: run_first[m], run_count[m] = the buckets launched by
 * that mark (run_count 0 if none). *n_launched = buckets launched in all.
 * Returns ORC_EINVAL if a parameter index is out of range or marked twice
 * (the source asserts that a ready bucket is never at or behind the next one
 * twice). */
int orc_reducer_schedule(const int32_t *bucket_of, int32_t n_params,
                         int32_t n_buckets, const int32_t *order,
                         int32_t n_marks, int32_t *run_first,
                         int32_t *run_count, int32_t *n_launched) {
  if (n_params < 0 || n_buckets < 0 || n_marks < 0) return ORC_EINVAL;
  int32_t *pending = (int32_t *)calloc((size_t)(n_buckets + 1), sizeof(int32_t));
  char *seen = (char *)calloc((size_t)(n_params + 1), 1);
  if (pending == NULL || seen == NULL) {
    free(pending);
    free(seen);
    return ORC_ENOMEM;
  }
  for (int32_t i = 0; i < n_params; ++i) pending[bucket_of[i]] += 1;
  int32_t next = 0;
  int rc = ORC_OK;
  for (int32_t m = 0; m < n_marks; ++m) {
    run_first[m] = next;
    run_count[m] = 0;
    int32_t i = order[m];
    if (i < 0 || i >= n_params || seen[i]) {
      rc = ORC_EINVAL;
      break;
    }
    seen[i] = 1;
    int32_t b = bucket_of[i];
    pending[b] -= 1;
    if (pending[b] == 0 && b == next) {
      while (next < n_buckets && pending[next] == 0) {
        next += 1;
        run_count[m] += 1;
      }
    }
  }
  *n_launched = next;
  free(pending);
  free(seen);
  return rc;
}

/* ------------------------------------------------------------------------ */
/* Logarithmic-latency all-reduce schedules                                  */
/* ------------------------------------------------------------------------ */

/* [DP] "Latency, trees, and choosing an algorithm" describes recursive
 * doubling and recursive halving/doubling for p a power of two. For any
 * other p the pages say nothing; the reading taken here (listed with the
 * other readings) is the usual one: with q the largest power of two <= p,
 * each "extra" rank r >= q first hands its whole buffer to rank r - q, which
 * adds it (FOLD_IN); the q core ranks run the schedule; then every extra
 * rank receives the finished result from rank r - q (FOLD_OUT). */
static int32_t pow2_floor(int32_t p) {
  int32_t q = 1;
  while (q * 2 <= p) q *= 2;
  return q;
}

/* Extra ranks fold into their partners (whole buffers, no send buffer
 * needed: senders r >= q are never receivers in this step). */
static void fold_in(float **work, int32_t p, int32_t q, int64_t len, int64_t n,
                    int64_t wire_bytes, msg_log *log) {
  for (int32_t r = q; r < p; ++r) {
    log_msg(log, ORC_PHASE_FOLD_IN, 0, r, r - q, -1, n * wire_bytes);
    for (int64_t i = 0; i < len; ++i) work[r - q][i] = work[r - q][i] + work[r][i];
  }
}

static void fold_out(float **work, int32_t p, int32_t q, int64_t len, int64_t n,
                     int32_t step, int64_t wire_bytes, msg_log *log) {
  for (int32_t r = q; r < p; ++r) {
    log_msg(log, ORC_PHASE_FOLD_OUT, step, r - q, r, -1, n * wire_bytes);
    memcpy(work[r], work[r - q], (size_t)len * sizeof(float));
  }
}

/* Recursive doubling: in step j every core rank r exchanges its whole
 * current buffer with rank r XOR 2^j and both add what they received. Each
 * step first copies every outgoing buffer, then delivers. After log2(q)
 * steps every core rank holds the sum, which it then divides. */
static void rd_on_work(float **work, float **send, int32_t p, int64_t n,
                       int32_t do_divide, float divisor, int64_t wire_bytes,
                       msg_log *log) {
  int32_t q = pow2_floor(p);
  int32_t step = 0;
  if (q < p) {
    fold_in(work, p, q, n, n, wire_bytes, log);
    step += 1;
  }
  for (int32_t d = 1; d < q; d *= 2, ++step) {
    for (int32_t r = 0; r < q; ++r) {
      memcpy(send[r], work[r], (size_t)n * sizeof(float));
      log_msg(log, ORC_PHASE_EXCHANGE, step, r, r ^ d, -1, n * wire_bytes);
    }
    for (int32_t r = 0; r < q; ++r) {
      const float *got = send[r ^ d];
      for (int64_t i = 0; i < n; ++i) work[r][i] = work[r][i] + got[i];
    }
  }
  if (do_divide) {
    for (int32_t r = 0; r < q; ++r) {
      for (int64_t i = 0; i < n; ++i) work[r][i] = work[r][i] / divisor;
    }
  }
  if (q < p) fold_out(work, p, q, n, n, step, wire_bytes, log);
}

/* Recursive halving, then recursive doubling (Rabenseifner). The padded
 * buffer is cut into q chunks of C = ceil(n/q). Halving step s = 1..log2(q)
 * pairs rank r with r XOR q/2^s: the two share a range of chunks; each keeps
 * the half whose chunk indices agree with its own rank in that bit, sends
 * the other half to its partner, and adds the half it receives. After the
 * last halving step rank r owns the finished chunk r, which it divides.
 * Doubling steps then run the pairings in reverse order (distance 1 first),
 * each rank sending everything it owns and storing what it receives, until
 * every core rank holds the whole buffer. */
static void rab_on_work(float **work, float **send, int32_t p, int64_t n,
                        int64_t C, int32_t do_divide, float divisor,
                        int64_t wire_bytes, msg_log *log) {
  int32_t q = pow2_floor(p);
  int64_t len = C * q;
  int32_t step = 0;
  if (q < p) {
    fold_in(work, p, q, len, n, wire_bytes, log);
    step += 1;
  }
  int64_t lo[64 + 1];
  for (int32_t r = 0; r < q; ++r) lo[r] = 0;
  int64_t cnt = q; /* chunks in each rank's current range */
  for (int32_t d = q / 2; d >= 1; d /= 2, ++step) {
    int64_t half = cnt / 2;
    for (int32_t r = 0; r < q; ++r) {
      int64_t give = (r & d) ? lo[r] : lo[r] + half;
      memcpy(send[r], work[r] + give * C, (size_t)(half * C) * sizeof(float));
      log_msg(log, ORC_PHASE_REDUCE_SCATTER, step, r, r ^ d, (int32_t)give,
              half * C * wire_bytes);
    }
    for (int32_t r = 0; r < q; ++r) {
      int64_t keep = (r & d) ? lo[r] + half : lo[r];
      float *mine = work[r] + keep * C;
      const float *got = send[r ^ d];
      for (int64_t i = 0; i < half * C; ++i) mine[i] = mine[i] + got[i];
    }
    for (int32_t r = 0; r < q; ++r) {
      if (r & d) lo[r] += half;
    }
    cnt = half;
  }
  if (do_divide) {
    for (int32_t r = 0; r < q; ++r) {
      float *mine = work[r] + lo[r] * C;
      for (int64_t i = 0; i < C; ++i) mine[i] = mine[i] / divisor;
    }
  }
  for (int32_t d = 1; d < q; d *= 2, ++step) {
    for (int32_t r = 0; r < q; ++r) {
      memcpy(send[r], work[r] + lo[r] * C, (size_t)(cnt * C) * sizeof(float));
      log_msg(log, ORC_PHASE_ALLGATHER, step, r, r ^ d, (int32_t)lo[r],
              cnt * C * wire_bytes);
    }
    for (int32_t r = 0; r < q; ++r) {
      memcpy(work[r] + lo[r ^ d] * C, send[r ^ d],
             (size_t)(cnt * C) * sizeof(float));
    }
    for (int32_t r = 0; r < q; ++r) {
      if (r & d) lo[r] -= cnt;
    }
    cnt *= 2;
  }
  if (q < p) fold_out(work, p, q, len, n, step, wire_bytes, log);
}

/* Tree all-reduce: reduce up the doubling tree to rank 0, then broadcast
 * down the same tree ([COL] exercise: a tree allreduce variant beside the
 * ring; its broadcast already uses the doubling tree). Reduction runs the
 * broadcast's rounds backwards: for span = 2^(K-1), ..., 2, 1 (K =
 * ceil(log2 p)) every rank v < span with v + span < p receives v + span's
 * buffer and adds it. Senders (v >= span) are never receivers in the same
 * round, so no send buffer is needed. Rank 0 divides the finished sum. */
static void tree_on_work(float **work, int32_t p, int64_t n, int32_t do_divide,
                         float divisor, int64_t wire_bytes, msg_log *log) {
  int32_t K = 0;
  while ((1 << K) < p) K += 1;
  int32_t step = 0;
  for (int32_t j = K - 1; j >= 0; --j, ++step) {
    int32_t span = 1 << j;
    for (int32_t v = 0; v < span; ++v) {
      if (v + span >= p) continue;
      log_msg(log, ORC_PHASE_REDUCE, step, v + span, v, -1, n * wire_bytes);
      for (int64_t i = 0; i < n; ++i) work[v][i] = work[v][i] + work[v + span][i];
    }
  }
  if (do_divide) {
    for (int64_t i = 0; i < n; ++i) work[0][i] = work[0][i] / divisor;
  }
  for (int32_t j = 0; j < K; ++j, ++step) {
    int32_t span = 1 << j;
    for (int32_t v = 0; v < span; ++v) {
      if (v + span >= p) continue;
      log_msg(log, ORC_PHASE_BROADCAST, step, v, v + span, -1, n * wire_bytes);
      memcpy(work[v + span], work[v], (size_t)n * sizeof(float));
    }
  }
}

/* All-reduce of p rank arrays of n elements, in place, under `schedule`
 * (ORC_SCHED_*). dtype, avg_mode, tokens, log, log_capacity and n_msgs as
 * for orc_ring_allreduce (which ORC_SCHED_RING runs). Every schedule's wire
 * carries fp32 values. */
int orc_allreduce(void *const *bufs, int32_t p, int64_t n, int32_t dtype,
                  int32_t avg_mode, const int64_t *tokens, int32_t schedule,
                  orc_msg *log, int64_t log_capacity, int64_t *n_msgs) {
  if (schedule == ORC_SCHED_RING) {
    return orc_ring_allreduce(bufs, p, n, dtype, avg_mode, tokens, -1, log,
                              log_capacity, n_msgs);
  }
  if (p < 1 || p > 64 || n < 0 || (dtype != 0 && dtype != 1)) return ORC_EINVAL;
  if (schedule < ORC_SCHED_RECURSIVE_DOUBLING || schedule > ORC_SCHED_TREE) {
    return ORC_EINVAL;
  }
  float divisor = 1.0f;
  int rc = avg_divisor(avg_mode, p, tokens, &divisor);
  if (rc != ORC_OK) return rc;
  int32_t q = pow2_floor(p);
  int64_t C = (n + q - 1) / q;
  int64_t len = schedule == ORC_SCHED_RABENSEIFNER ? C * q : n;
  float **work = alloc_arrays(p, len);
  float **send = alloc_arrays(p, len);
  if (work == NULL || send == NULL) {
    free_arrays(work, p);
    free_arrays(send, p);
    return ORC_ENOMEM;
  }
  for (int32_t r = 0; r < p; ++r) {
    if (dtype == 0) {
      memcpy(work[r], bufs[r], (size_t)n * sizeof(float));
    } else {
      orc_bf16_to_f32_array((const uint16_t *)bufs[r], work[r], n);
    }
  }
  msg_log lg = {log, log_capacity, 0};
  int32_t do_divide = avg_mode != ORC_AVG_NONE;
  int64_t wire = (int64_t)sizeof(float);
  if (schedule == ORC_SCHED_RECURSIVE_DOUBLING) {
    rd_on_work(work, send, p, n, do_divide, divisor, wire, &lg);
  } else if (schedule == ORC_SCHED_RABENSEIFNER) {
    rab_on_work(work, send, p, n, C, do_divide, divisor, wire, &lg);
  } else {
    tree_on_work(work, p, n, do_divide, divisor, wire, &lg);
  }
  for (int32_t r = 0; r < p; ++r) {
    if (dtype == 0) {
      memcpy(bufs[r], work[r], (size_t)n * sizeof(float));
    } else {
      orc_f32_to_bf16_array(work[r], (uint16_t *)bufs[r], n);
    }
  }
  if (n_msgs != NULL) *n_msgs = lg.count;
  free_arrays(work, p);
  free_arrays(send, p);
  return ORC_OK;
}

/* The value the logarithmic schedules reach at one element, as a pairwise
 * fold of that element's p values (vals[s*p + r] = rank r's value for
 * sample s). With q the largest power of two <= p, leaf v < q is
 * x[v] + x[v+q] when rank v+q exists, else x[v]. Then pairs of partial sums
 * combine level by level:
 *   recursive doubling   distance 1 first: (leaf 0 + leaf 1), (2 + 3), ...
 *                        then those pairs at distance 2, and so on;
 *   Rabenseifner, tree   distance q/2 first: (leaf 0 + leaf q/2), ... then
 *                        q/4, and so on.
 * Every rank of a pair computes a + b or b + a, the same number, so the
 * pairing alone fixes the result. Derived from the exchanges each schedule
 * performs; pinned to the literal simulations in tests. */
int32_t orc_tree_fold_samples(const float *vals, int32_t p, int64_t count,
                              int32_t schedule, int32_t do_divide, float divisor,
                              float *out) {
  /* the partial sums of one element live in t[]: at most 64 ranks */
  if (p < 1 || p > 64 || count < 0) return ORC_EINVAL;
  int32_t q = pow2_floor(p);
  float t[64];
  for (int64_t s = 0; s < count; ++s) {
    const float *x = vals + s * p;
    for (int32_t v = 0; v < q; ++v) t[v] = v + q < p ? x[v] + x[v + q] : x[v];
    if (schedule == ORC_SCHED_RECURSIVE_DOUBLING) {
      for (int32_t d = 1; d < q; d *= 2) {
        for (int32_t v = 0; v < q; v += 2 * d) t[v] = t[v] + t[v + d];
      }
    } else {
      for (int32_t d = q / 2; d >= 1; d /= 2) {
        for (int32_t v = 0; v < d; ++v) t[v] = t[v] + t[v + d];
      }
    }
    out[s] = do_divide ? t[0] / divisor : t[0];
  }
  return ORC_OK;
}

/* ------------------------------------------------------------------------ */
/* Coalesced broadcast of many tensors                                       */
/* ------------------------------------------------------------------------ */

/* Broadcast n_t tensors from rank `root` to every rank, coalesced ("PyTorch
 * DDP Deep Dive", Part 1, the init-time broadcast of parameters and buffers,
 * and Part 2, the per-forward buffer broadcast): the tensors are grouped by
 * orc_coalesce_plan; for each bucket the root's tensors are flattened into
 * one buffer, that buffer is broadcast over the doubling tree (as
 * orc_broadcast, relative to the root), and every rank unflattens it into
 * its own tensors. tensors[r * n_t + i] is rank r's copy of tensor i, of
 * numel[i] elements of elem_bytes bytes. Logged messages carry the bucket
 * number in `chunk`. bucket_of (may be NULL) receives each tensor's bucket. */
int orc_broadcast_coalesced(void *const *tensors, const int64_t *numel,
                            int32_t n_t, int32_t p, int32_t elem_bytes,
                            int64_t cap, int32_t root, orc_msg *log,
                            int64_t log_capacity, int64_t *n_msgs,
                            int32_t *bucket_of) {
  if (p < 1 || n_t < 0 || elem_bytes <= 0 || root < 0 || root >= p) {
    return ORC_EINVAL;
  }
  int32_t m = n_t > 0 ? n_t : 1;
  int32_t *fill = (int32_t *)calloc((size_t)m, sizeof(int32_t));
  int32_t *begin = (int32_t *)calloc((size_t)m + 1, sizeof(int32_t));
  int64_t *off = (int64_t *)calloc((size_t)m, sizeof(int64_t));
  int32_t *bof = (int32_t *)calloc((size_t)m, sizeof(int32_t));
  char **flat = (char **)calloc((size_t)p, sizeof(char *));
  int rc = ORC_OK;
  int32_t nb = 0;
  if (fill == NULL || begin == NULL || off == NULL || bof == NULL || flat == NULL) {
    rc = ORC_ENOMEM;
  } else {
    rc = orc_coalesce_plan(numel, n_t, elem_bytes, cap, fill, begin, off, bof, &nb);
  }
  msg_log lg = {log, log_capacity, 0};
  int32_t round = 0;
  for (int32_t b = 0; b < nb && rc == ORC_OK; ++b) {
    int64_t bytes = 0;
    for (int32_t k = begin[b]; k < begin[b + 1]; ++k) bytes += numel[fill[k]] * elem_bytes;
    for (int32_t r = 0; r < p && rc == ORC_OK; ++r) {
      flat[r] = (char *)calloc((size_t)bytes + 1, 1);
      if (flat[r] == NULL) rc = ORC_ENOMEM;
    }
    if (rc == ORC_OK) {
      /* the root flattens its tensors */
      for (int32_t k = begin[b]; k < begin[b + 1]; ++k) {
        int32_t i = fill[k];
        memcpy(flat[root] + off[i] * elem_bytes, tensors[(int64_t)root * n_t + i],
               (size_t)(numel[i] * elem_bytes));
      }
      /* doubling tree on relative rank v = (r - root) mod p */
      for (int64_t span = 1; span < p; span *= 2, ++round) {
        for (int64_t v = 0; v < span; ++v) {
          if (v + span >= p) continue;
          int32_t s = (int32_t)((v + root) % p);
          int32_t d = (int32_t)((v + span + root) % p);
          memcpy(flat[d], flat[s], (size_t)bytes);
          log_msg(&lg, ORC_PHASE_BROADCAST, round, s, d, b, bytes);
        }
      }
      /* every rank unflattens */
      for (int32_t r = 0; r < p; ++r) {
        for (int32_t k = begin[b]; k < begin[b + 1]; ++k) {
          int32_t i = fill[k];
          memcpy(tensors[(int64_t)r * n_t + i], flat[r] + off[i] * elem_bytes,
                 (size_t)(numel[i] * elem_bytes));
        }
      }
    }
    for (int32_t r = 0; r < p; ++r) {
      free(flat[r]);
      flat[r] = NULL;
    }
  }
  if (rc == ORC_OK) {
    if (n_msgs != NULL) *n_msgs = lg.count;
    if (bucket_of != NULL) {
      for (int32_t i = 0; i < n_t; ++i) bucket_of[i] = bof[i];
    }
  }
  free(fill);
  free(begin);
  free(off);
  free(bof);
  free(flat);
  return rc;
}
