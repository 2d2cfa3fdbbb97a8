// Host-side entry points of libddpsim under AddressSanitizer and
// UndefinedBehaviorSanitizer (the planner, the piece-table builder, the
// coalescing planner, the overlap model and argument errors; no GPU work).
// Built by tests/test_c_abi.py with the host sources instrumented; prints
// "ok <checks>" and exits 0 when every invariant held.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <utility>
#include <vector>

#include "ddpsim.h"

namespace {

uint64_t g_state = 0x9E3779B97F4A7C15ull;
uint64_t next() {  // xorshift64*
  g_state ^= g_state >> 12;
  g_state ^= g_state << 25;
  g_state ^= g_state >> 27;
  return g_state * 0x2545F4914F6CDD1Dull;
}
int64_t uniform(int64_t lo, int64_t hi) {  // [lo, hi]
  return lo + static_cast<int64_t>(next() % static_cast<uint64_t>(hi - lo + 1));
}

long g_checks = 0;
#define CHECK(cond)                                                     \
  do {                                                                  \
    ++g_checks;                                                         \
    if (!(cond)) {                                                      \
      std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
      std::exit(1);                                                     \
    }                                                                   \
  } while (0)

// Every parameter in exactly one bucket at the offset its bucket's earlier
// members leave; bucket sizes and element counts consistent.
void check_plan(const ddp_plan *plan, const std::vector<int64_t> &numel) {
  const int32_t n = static_cast<int32_t>(numel.size());
  CHECK(ddp_plan_num_params(plan) == n);
  const int32_t nb = ddp_plan_num_buckets(plan);
  CHECK(nb >= (n > 0 ? 1 : 0));
  std::vector<int> seen(static_cast<size_t>(n), 0);
  for (int32_t b = 0; b < nb; ++b) {
    const int32_t k = ddp_plan_bucket_size(plan, b);
    CHECK(k >= 1);
    std::vector<int32_t> idx(static_cast<size_t>(k));
    CHECK(ddp_plan_bucket_params(plan, b, idx.data()) == DDP_OK);
    int64_t off = 0;
    for (int32_t i : idx) {
      CHECK(i >= 0 && i < n);
      seen[static_cast<size_t>(i)] += 1;
      CHECK(ddp_plan_param_bucket(plan, i) == b);
      CHECK(ddp_plan_param_offset(plan, i) == off);
      off += numel[static_cast<size_t>(i)];
    }
    CHECK(ddp_plan_bucket_numel(plan, b) == off);
  }
  for (int s : seen) CHECK(s == 1);
  CHECK(ddp_plan_bucket_size(plan, nb) == -1);
  CHECK(ddp_plan_bucket_numel(plan, -1) == -1);
  CHECK(ddp_plan_param_bucket(plan, n) == -1);
  CHECK(ddp_plan_device_bytes(plan) >= static_cast<size_t>(32) * n);
}

}  // namespace

int main() {
  for (int iter = 0; iter < 1500; ++iter) {
    const int32_t n = static_cast<int32_t>(uniform(0, 120));
    std::vector<int64_t> numel(static_cast<size_t>(n));
    for (auto &v : numel) v = next() % 5 == 0 ? uniform(0, 3) : uniform(0, 70000);
    const int32_t eb = next() % 2 ? 4 : 2;
    const int64_t cap = uniform(0, 300000);
    const int64_t first = uniform(0, 100000);

    ddp_plan *plan = nullptr;
    CHECK(ddp_bucket_plan(numel.data(), n, eb, cap, first, &plan) == DDP_OK);
    check_plan(plan, numel);
    // the piece table of the in-place all-reduce, for several rank counts
    int64_t total = 0;
    for (int64_t v : numel) total += v;
    for (int t = 0; t < 3; ++t) {
      const int32_t p = static_cast<int32_t>(uniform(1, 64));
      const size_t bytes = ddp_plan_segment_bytes(plan, p);
      CHECK((bytes > 0) == (total > 0));  // zero-size parameters have no pieces
    }
    // the overlap model on random times
    const int32_t nb = ddp_plan_num_buckets(plan);
    std::vector<double> ready(static_cast<size_t>(n)), bt(static_cast<size_t>(nb) + 1);
    double last = 0.0;
    for (auto &r : ready) {
      r = static_cast<double>(uniform(0, 1000)) * 1e-4;
      last = r > last ? r : last;
    }
    for (auto &b : bt) b = static_cast<double>(uniform(0, 1000)) * 1e-5;
    double step = -1.0, exposed = -1.0;
    CHECK(ddp_overlap_step_time(plan, ready.data(), bt.data(), &step, &exposed) == DDP_OK);
    CHECK(step >= last && exposed >= 0.0 && std::fabs(step - exposed - last) <= 1e-12);
    ddp_plan_free(plan);

    // the same bucketing over a random walk order, and a walk that repeats
    std::vector<int32_t> order(static_cast<size_t>(n));
    for (int32_t i = 0; i < n; ++i) order[static_cast<size_t>(i)] = i;
    for (int32_t i = n - 1; i > 0; --i) {
      std::swap(order[static_cast<size_t>(i)], order[static_cast<size_t>(uniform(0, i))]);
    }
    CHECK(ddp_bucket_plan_ordered(numel.data(), n, order.data(), eb, cap, first, &plan) ==
          DDP_OK);
    check_plan(plan, numel);
    ddp_plan_free(plan);
    if (n >= 2) {
      order[0] = order[1];
      plan = reinterpret_cast<ddp_plan *>(&order);  // must be reset to NULL on error
      CHECK(ddp_bucket_plan_ordered(numel.data(), n, order.data(), eb, cap, first, &plan) ==
            DDP_EINVAL);
      CHECK(plan == nullptr);
    }

    // coalescing planner: no bucket past the cap unless one tensor alone is
    const int32_t ceb = 1 << uniform(0, 3);
    const int64_t ccap = uniform(1, 400000);
    CHECK(ddp_coalesce_plan(numel.data(), n, ceb, ccap, &plan) == DDP_OK);
    check_plan(plan, numel);
    for (int32_t b = 0; b < ddp_plan_num_buckets(plan); ++b) {
      CHECK(ddp_plan_bucket_numel(plan, b) * ceb <= ccap || ddp_plan_bucket_size(plan, b) == 1);
    }
    ddp_plan_free(plan);
  }

  // argument errors: nothing is allocated, *out is cleared
  const int64_t bad[3] = {5, -1, 7};
  ddp_plan *plan = nullptr;
  CHECK(ddp_bucket_plan(bad, 3, 4, 100, 10, &plan) == DDP_EINVAL && plan == nullptr);
  CHECK(ddp_bucket_plan(bad, 1, 3, 100, 10, &plan) == DDP_EINVAL);
  CHECK(ddp_bucket_plan(bad, 1, 4, -1, 10, &plan) == DDP_EINVAL);
  CHECK(ddp_bucket_plan(nullptr, 2, 4, 100, 10, &plan) == DDP_EINVAL);
  CHECK(ddp_bucket_plan(bad, 1, 4, 100, 10, nullptr) == DDP_EINVAL);
  CHECK(ddp_coalesce_plan(bad, 1, 3, 100, &plan) == DDP_EINVAL);
  CHECK(ddp_overlap_step_time(nullptr, nullptr, nullptr, nullptr, nullptr) == DDP_EINVAL);
  CHECK(ddp_last_error()[0] != '\0');
  // a reducer needs the piece table for its p
  CHECK(ddp_bucket_plan(bad, 1, 4, 100, 10, &plan) == DDP_OK);
  ddp_reducer *red = nullptr;
  CHECK(ddp_reducer_create(plan, 4, nullptr, DDP_F32, DDP_AVG_WORLD, nullptr, nullptr, &red) !=
        DDP_OK);
  CHECK(red == nullptr);
  ddp_plan_free(plan);
  std::printf("ok %ld\n", g_checks);
  return 0;
}
