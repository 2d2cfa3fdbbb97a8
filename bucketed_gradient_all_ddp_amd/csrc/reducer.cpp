// reducer.cpp -- readiness bookkeeping that launches bucket all-reduces as
// backward produces gradients ("PyTorch DDP Deep Dive", Part 2 "Step 2:
// backward" and "Step 3: finalize_backward"; "Data parallelism", section
// "Overlapping communication with the backward pass").
//
// Every bucket starts a backward pass with a pending count equal to its
// number of parameters. A ready mark decrements the count of the
// parameter's bucket; when that count reaches zero and the bucket is the
// next one to reduce, the reducer launches it and every following bucket
// that is already complete, as one run (ddp_allreduce_buckets), on the
// communication stream, after making that stream wait for the events the
// producers attached to those buckets' parameters. Buckets therefore start
// in index order, each as early as its own gradients and its predecessors
// allow, overlapping whatever the producer streams still compute.
// finalize() reports a bucket that never became ready instead of waiting for
// it forever. The order of the marks is kept, so the buckets can be rebuilt
// from the order in which gradients actually became ready (Part 2: the hook
// records each ready parameter while a rebuild is due, and the rebuild runs
// before the next forward).
#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <new>
#include <vector>

#include "internal.hpp"

namespace ddpsim {
bool plan_segment_info(const ddp_plan *plan, int32_t b, int32_t *first, int32_t *count,
                       int32_t *tiles, int32_t *tile_first, int64_t *elems,
                       const void **table, int32_t *seg_p, int32_t *n_params,
                       int32_t *elem_bytes);
}  // namespace ddpsim

using namespace ddpsim;

struct ddp_reducer {
  const ddp_plan *plan = nullptr;
  int32_t p = 0;
  int32_t dtype = 0;
  int32_t avg_mode = 0;
  std::vector<int64_t> tokens;
  void *const *grads = nullptr;
  hipStream_t comm = nullptr;
  std::vector<int32_t> bucket_of;   // per parameter
  std::vector<int32_t> size;        // parameters per bucket
  std::vector<int32_t> pending;     // per bucket, this pass
  std::vector<char> ready;          // per parameter, this pass
  std::vector<std::vector<hipEvent_t>> events;  // per bucket, this pass
  int32_t next = 0;
  int32_t marks = 0;
  int32_t max_workgroups = 0;  // cap on each launch's workgroups (0: none)
  bool active = false;
  std::vector<int32_t> log_mark, log_first, log_count;
  std::vector<int32_t> ready_order;  // parameters in the order marked, this pass
  hipEvent_t done = nullptr;
  // A launch that failed during this pass: every later call of the pass
  // (marks and finalize) reports it, so the cause is not hidden behind
  // buckets that then look as if they never became ready.
  ddp_status failed = DDP_OK;
  char failed_detail[512] = "";
};

extern "C" ddp_status ddp_reducer_create(const ddp_plan *plan, int32_t p,
                                         void *const *d_grad_ptrs, int32_t dtype,
                                         int32_t avg_mode, const int64_t *tokens,
                                         hipStream_t comm_stream, ddp_reducer **out) {
  clear_error();
  const char *what = "ddp_reducer_create";
  if (out == nullptr) return fail(DDP_EINVAL, "%s: out is NULL", what);
  *out = nullptr;
  if (plan == nullptr) return fail(DDP_EINVAL, "%s: plan is NULL", what);
  ddp_status s = check_p(p, what);
  if (s != DDP_OK) return s;
  const int32_t n_params = ddp_plan_num_params(plan);
  const int32_t n_buckets = ddp_plan_num_buckets(plan);
  int32_t f, c, t, tf, seg_p, np, eb_plan = 0;
  int64_t e;
  const void *table;
  if (n_buckets > 0) {
    plan_segment_info(plan, 0, &f, &c, &t, &tf, &e, &table, &seg_p, &np, &eb_plan);
  }
  const int eb = elem_bytes_of(dtype);
  if (eb == 0) return fail(DDP_EINVAL, "%s: unknown dtype %d", what, dtype);
  if (n_buckets > 0 && eb != eb_plan) {
    return fail(DDP_EINVAL, "%s: dtype has %d-byte elements, the plan %d", what, eb, eb_plan);
  }
  if (n_buckets > 0 && seg_p != p) {
    return fail(DDP_ENOTREADY, "%s: call ddp_plan_upload_segments with p=%d first", what, p);
  }
  if (n_params > 0 && d_grad_ptrs == nullptr) {
    return fail(DDP_EINVAL, "%s: gradient pointer table is NULL", what);
  }
  Divide div;
  s = make_divide(avg_mode, p, tokens, &div);
  if (s != DDP_OK) return s;
  ddp_reducer *r = new (std::nothrow) ddp_reducer;
  if (r == nullptr) return fail(DDP_EINVAL, "%s: out of host memory", what);
  r->plan = plan;
  r->p = p;
  r->dtype = dtype;
  r->avg_mode = avg_mode;
  if (avg_mode == DDP_AVG_TOKENS) r->tokens.assign(tokens, tokens + p);
  r->grads = d_grad_ptrs;
  r->comm = comm_stream;
  r->bucket_of.resize(n_params);
  for (int32_t i = 0; i < n_params; ++i) r->bucket_of[i] = ddp_plan_param_bucket(plan, i);
  r->size.resize(n_buckets);
  for (int32_t b = 0; b < n_buckets; ++b) r->size[b] = ddp_plan_bucket_size(plan, b);
  *out = r;
  return DDP_OK;
}

extern "C" void ddp_reducer_free(ddp_reducer *r) {
  if (r == nullptr) return;
  if (r->done != nullptr) (void)hipEventDestroy(r->done);
  delete r;
}

extern "C" ddp_status ddp_reducer_set_max_workgroups(ddp_reducer *r, int32_t max_workgroups) {
  clear_error();
  if (r == nullptr) return fail(DDP_EINVAL, "ddp_reducer_set_max_workgroups: reducer is NULL");
  if (max_workgroups < 0) {
    return fail(DDP_EINVAL, "ddp_reducer_set_max_workgroups: %d is negative", max_workgroups);
  }
  r->max_workgroups = max_workgroups;
  return DDP_OK;
}

extern "C" ddp_status ddp_reducer_prepare(ddp_reducer *r) {
  clear_error();
  if (r == nullptr) return fail(DDP_EINVAL, "ddp_reducer_prepare: reducer is NULL");
  r->pending = r->size;
  r->ready.assign(r->bucket_of.size(), 0);
  r->events.assign(r->size.size(), {});
  r->next = 0;
  r->marks = 0;
  r->log_mark.clear();
  r->log_first.clear();
  r->log_count.clear();
  r->ready_order.clear();
  r->failed = DDP_OK;
  r->failed_detail[0] = '\0';
  r->active = true;
  return DDP_OK;
}

namespace {

// The sticky launch failure of the pass, reported again by `what`.
ddp_status report_failure(const ddp_reducer *r, const char *what) {
  return fail(r->failed, "%s: an earlier launch of this pass failed: %s", what,
              r->failed_detail);
}

}  // namespace

extern "C" ddp_status ddp_reducer_mark_ready(ddp_reducer *r, int32_t param,
                                             hipEvent_t ready) {
  clear_error();
  const char *what = "ddp_reducer_mark_ready";
  if (r == nullptr) return fail(DDP_EINVAL, "%s: reducer is NULL", what);
  if (!r->active) return fail(DDP_EINVAL, "%s: call ddp_reducer_prepare first", what);
  if (r->failed != DDP_OK) return report_failure(r, what);
  if (param < 0 || param >= static_cast<int32_t>(r->bucket_of.size())) {
    return fail(DDP_ERANGE, "%s: parameter %d out of range", what, param);
  }
  if (r->ready[param]) {
    return fail(DDP_EINVAL, "%s: parameter %d marked ready twice in one pass", what, param);
  }
  r->ready[param] = 1;
  r->ready_order.push_back(param);
  const int32_t b = r->bucket_of[param];
  if (ready != nullptr &&
      std::find(r->events[b].begin(), r->events[b].end(), ready) == r->events[b].end()) {
    r->events[b].push_back(ready);
  }
  r->pending[b] -= 1;
  const int32_t mark = r->marks++;
  const int32_t n_buckets = static_cast<int32_t>(r->size.size());
  if (r->pending[b] != 0 || b != r->next) return DDP_OK;
  int32_t end = r->next;
  while (end < n_buckets && r->pending[end] == 0) ++end;
  ddp_status s = DDP_OK;
  for (int32_t k = r->next; k < end && s == DDP_OK; ++k) {
    for (hipEvent_t ev : r->events[k]) {
      s = check_hip(hipStreamWaitEvent(r->comm, ev, 0), "hipStreamWaitEvent");
      if (s != DDP_OK) break;
    }
  }
  if (s == DDP_OK) {
    s = allreduce_buckets(r->plan, r->next, end - r->next, r->p, r->grads, r->dtype,
                          r->avg_mode, r->tokens.empty() ? nullptr : r->tokens.data(), r->comm,
                          nullptr, r->max_workgroups);
  }
  if (s != DDP_OK) {
    r->failed = s;
    std::snprintf(r->failed_detail, sizeof r->failed_detail, "buckets %d..%d: %s", r->next,
                  end - 1, ddp_last_error());
    return fail(s, "%s: %s", what, r->failed_detail);
  }
  r->log_mark.push_back(mark);
  r->log_first.push_back(r->next);
  r->log_count.push_back(end - r->next);
  r->next = end;
  return DDP_OK;
}

extern "C" ddp_status ddp_reducer_finalize(ddp_reducer *r, hipStream_t wait_stream) {
  clear_error();
  const char *what = "ddp_reducer_finalize";
  if (r == nullptr) return fail(DDP_EINVAL, "%s: reducer is NULL", what);
  if (!r->active) return fail(DDP_EINVAL, "%s: no backward pass in progress", what);
  r->active = false;
  if (r->failed != DDP_OK) return report_failure(r, what);
  const int32_t n_buckets = static_cast<int32_t>(r->size.size());
  if (r->next < n_buckets) {
    int32_t missing = 0;
    for (int32_t i = 0; i < static_cast<int32_t>(r->bucket_of.size()); ++i) {
      if (!r->ready[i]) ++missing;
    }
    return fail(DDP_ENOTREADY,
                "%s: bucket %d never became ready (%d of its %d parameters are still "
                "pending; %d parameters unmarked in all); buckets %d..%d were not reduced",
                what, r->next, r->pending[r->next], r->size[r->next], missing, r->next,
                n_buckets - 1);
  }
  if (wait_stream == r->comm) return DDP_OK;
  if (r->done == nullptr) {
    ddp_status s = check_hip(hipEventCreateWithFlags(&r->done, hipEventDisableTiming),
                             "hipEventCreateWithFlags");
    if (s != DDP_OK) return s;
  }
  ddp_status s = check_hip(hipEventRecord(r->done, r->comm), "hipEventRecord");
  if (s != DDP_OK) return s;
  return check_hip(hipStreamWaitEvent(wait_stream, r->done, 0), "hipStreamWaitEvent");
}

extern "C" int32_t ddp_reducer_launch_log(const ddp_reducer *r, int32_t *at_mark,
                                          int32_t *first_bucket, int32_t *n_buckets,
                                          int32_t capacity) {
  if (r == nullptr) return -1;
  const int32_t n = static_cast<int32_t>(r->log_mark.size());
  for (int32_t k = 0; k < n && k < capacity; ++k) {
    if (at_mark) at_mark[k] = r->log_mark[k];
    if (first_bucket) first_bucket[k] = r->log_first[k];
    if (n_buckets) n_buckets[k] = r->log_count[k];
  }
  return n;
}

extern "C" int32_t ddp_reducer_ready_order(const ddp_reducer *r, int32_t *order,
                                           int32_t capacity) {
  if (r == nullptr) return -1;
  const int32_t n = static_cast<int32_t>(r->ready_order.size());
  for (int32_t k = 0; k < n && k < capacity && order != nullptr; ++k) order[k] = r->ready_order[k];
  return n;
}

// The reducer's schedule in the latency-bandwidth model: bucket b starts at
// max(its last parameter's ready time, end of bucket b-1).
extern "C" ddp_status ddp_overlap_step_time(const ddp_plan *plan, const double *ready,
                                            const double *bucket_time, double *step,
                                            double *exposed) {
  clear_error();
  const char *what = "ddp_overlap_step_time";
  if (plan == nullptr) return fail(DDP_EINVAL, "%s: plan is NULL", what);
  const int32_t n_params = ddp_plan_num_params(plan);
  const int32_t n_buckets = ddp_plan_num_buckets(plan);
  if ((n_params > 0 && ready == nullptr) || (n_buckets > 0 && bucket_time == nullptr)) {
    return fail(DDP_EINVAL, "%s: ready or bucket_time is NULL", what);
  }
  for (int32_t i = 0; i < n_params; ++i) {
    if (!std::isfinite(ready[i]) || ready[i] < 0.0) {
      return fail(DDP_EINVAL, "%s: ready[%d] = %g is not a finite time >= 0", what, i, ready[i]);
    }
  }
  for (int32_t b = 0; b < n_buckets; ++b) {
    if (!std::isfinite(bucket_time[b]) || bucket_time[b] < 0.0) {
      return fail(DDP_EINVAL, "%s: bucket_time[%d] = %g is not a finite time >= 0", what, b,
                  bucket_time[b]);
    }
  }
  std::vector<double> bucket_ready(static_cast<size_t>(n_buckets), 0.0);
  double end_bwd = 0.0;
  for (int32_t i = 0; i < n_params; ++i) {
    const int32_t b = ddp_plan_param_bucket(plan, i);
    bucket_ready[static_cast<size_t>(b)] = std::max(bucket_ready[static_cast<size_t>(b)], ready[i]);
    end_bwd = std::max(end_bwd, ready[i]);
  }
  double finish = 0.0;
  for (int32_t b = 0; b < n_buckets; ++b) {
    finish = std::max(bucket_ready[static_cast<size_t>(b)], finish) + bucket_time[b];
  }
  const double t = std::max(end_bwd, finish);
  if (step != nullptr) *step = t;
  if (exposed != nullptr) *exposed = t - end_bwd;
  return DDP_OK;
}
