/* A plain C caller of libddpsim.so's host-side entry points (no GPU work):
 * plans the GPT-2-small gradient buckets, prices and chooses all-reduce
 * schedules, and reports errors. Built and run by tests/test_c_abi.py. */
#include <stdint.h>
#include <stdio.h>

#include "ddpsim.h"

int main(void) {
  /* GPT-2 small in registration order: wte, wpe, 12 layers, ln_f */
  int64_t numel[148];
  int n = 0;
  numel[n++] = 50257LL * 768;
  numel[n++] = 1024LL * 768;
  for (int l = 0; l < 12; ++l) {
    numel[n++] = 768; numel[n++] = 768;             /* ln_1 */
    numel[n++] = 768LL * 2304; numel[n++] = 2304;   /* c_attn */
    numel[n++] = 768LL * 768; numel[n++] = 768;     /* attn c_proj */
    numel[n++] = 768; numel[n++] = 768;             /* ln_2 */
    numel[n++] = 768LL * 3072; numel[n++] = 3072;   /* c_fc */
    numel[n++] = 3072LL * 768; numel[n++] = 768;    /* mlp c_proj */
  }
  numel[n++] = 768; numel[n++] = 768;               /* ln_f */
  ddp_plan *plan = NULL;
  if (ddp_bucket_plan(numel, n, 4, 25LL << 20, 1LL << 20, &plan) != DDP_OK) {
    fprintf(stderr, "plan: %s\n", ddp_last_error());
    return 1;
  }
  printf("params %d buckets %d\n", ddp_plan_num_params(plan), ddp_plan_num_buckets(plan));
  for (int b = 0; b < ddp_plan_num_buckets(plan); ++b) {
    printf("bucket %d size %d numel %lld\n", b, ddp_plan_bucket_size(plan, b),
           (long long)ddp_plan_bucket_numel(plan, b));
  }
  ddp_plan_free(plan);
  /* the ring / recursive-doubling crossover at 10 us and 50 GB/s, p = 8 */
  const double alpha = 10e-6, beta = 1.0 / 50e9;
  /* the overlapped step time on that network: 25 MiB buckets (the first one
   * too), parameter i ready (n - i) ms into backward */
  if (ddp_bucket_plan(numel, n, 4, 25LL << 20, 25LL << 20, &plan) != DDP_OK) return 1;
  double ready[148], btime[148], step = 0.0, exposed = 0.0;
  for (int i = 0; i < n; ++i) ready[i] = (n - i) * 1e-3;
  for (int b = 0; b < ddp_plan_num_buckets(plan); ++b) {
    btime[b] = ddp_schedule_time(DDP_SCHED_RING, 8, 4.0 * ddp_plan_bucket_numel(plan, b),
                                 alpha, beta);
  }
  if (ddp_overlap_step_time(plan, ready, btime, &step, &exposed) != DDP_OK) return 1;
  printf("overlap %.17g %.17g\n", step, exposed);
  ddp_plan_free(plan);
  const uint32_t ring_rd = (1u << DDP_SCHED_RING) | (1u << DDP_SCHED_RECURSIVE_DOUBLING);
  printf("choose 4.3MB %d 4.5MB %d\n", ddp_choose_schedule(8, 4300000, alpha, beta, ring_rd),
         ddp_choose_schedule(8, 4500000, alpha, beta, ring_rd));
  /* an error path: a negative size is reported, nothing is planned */
  int64_t bad[2] = {5, -1};
  ddp_status s = ddp_bucket_plan(bad, 2, 4, 100, 10, &plan);
  printf("error %d %s\n", (int)s, ddp_strerror(s));
  return 0;
}
