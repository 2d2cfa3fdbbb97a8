// host.cpp -- error reporting, argument validation and averaging set-up
// shared by every entry point of libddpsim.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <vector>

#include "internal.hpp"

namespace ddpsim {

namespace {
thread_local char g_last_error[512] = "";
thread_local hipEvent_t g_timer_start = nullptr;
thread_local hipEvent_t g_timer_stop = nullptr;
}

CallTimer CallTimer::take() {
  CallTimer t;
  t.start = g_timer_start;
  t.stop = g_timer_stop;
  g_timer_start = nullptr;
  g_timer_stop = nullptr;
  return t;
}

void clear_error() { g_last_error[0] = '\0'; }

ddp_status fail(ddp_status s, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
  va_end(ap);
  return s;
}

ddp_status check_hip(hipError_t e, const char *what) {
  if (e == hipSuccess) return DDP_OK;
  return fail(DDP_EHIP, "%s: %s", what, hipGetErrorString(e));
}

int elem_bytes_of(int32_t dtype) {
  if (dtype == DDP_F32) return 4;
  if (dtype == DDP_BF16) return 2;
  return 0;
}

ddp_status check_p(int32_t p, const char *what) {
  if (p < 1 || p > kMaxRanks) {
    return fail(DDP_ERANGE, "%s: p=%d outside [1, %d]", what, p, kMaxRanks);
  }
  return DDP_OK;
}

bool ranges_overlap(const void *a, int64_t na, const void *b, int64_t nb) {
  if (na <= 0 || nb <= 0) return false;
  auto x = reinterpret_cast<uintptr_t>(a);
  auto y = reinterpret_cast<uintptr_t>(b);
  return x < y + static_cast<uintptr_t>(nb) && y < x + static_cast<uintptr_t>(na);
}

bool all_vec_aligned(const void *const *bufs, int32_t p) {
  for (int32_t r = 0; r < p; ++r) {
    if (reinterpret_cast<uintptr_t>(bufs[r]) % kVecBytes != 0) return false;
  }
  return true;
}

ddp_status check_rank_buffers(const char *what, const void *const *bufs,
                              int32_t p, int64_t bytes, int align) {
  if (bufs == nullptr) return fail(DDP_EINVAL, "%s: pointer array is NULL", what);
  if (bytes == 0) return DDP_OK;
  std::vector<std::pair<uintptr_t, int32_t>> order;
  order.reserve(p);
  for (int32_t r = 0; r < p; ++r) {
    if (bufs[r] == nullptr) {
      return fail(DDP_EINVAL, "%s: buffer of rank %d is NULL", what, r);
    }
    auto a = reinterpret_cast<uintptr_t>(bufs[r]);
    if (a % static_cast<uintptr_t>(align) != 0) {
      return fail(DDP_EALIGN, "%s: buffer of rank %d is not %d-byte aligned",
                  what, r, align);
    }
    order.emplace_back(a, r);
  }
  std::sort(order.begin(), order.end());
  for (size_t k = 1; k < order.size(); ++k) {
    if (order[k].first < order[k - 1].first + static_cast<uintptr_t>(bytes)) {
      return fail(DDP_EALIAS, "%s: buffers of ranks %d and %d overlap", what,
                  order[k - 1].second, order[k].second);
    }
  }
  return DDP_OK;
}

ddp_status make_divide(int32_t avg_mode, int32_t p, const int64_t *tokens,
                       Divide *out) {
  double divisor = 1.0;
  if (avg_mode == DDP_AVG_NONE) {
    divisor = 1.0;
  } else if (avg_mode == DDP_AVG_WORLD) {
    divisor = p;
  } else if (avg_mode == DDP_AVG_TOKENS) {
    if (tokens == nullptr) {
      return fail(DDP_EINVAL, "token averaging needs the per-rank token counts");
    }
    int64_t total = 0;
    for (int32_t r = 0; r < p; ++r) {
      if (tokens[r] < 0) {
        return fail(DDP_EINVAL, "token count of rank %d is negative", r);
      }
      if (tokens[r] > (INT64_MAX >> 8)) {
        return fail(DDP_EINVAL, "token count of rank %d is too large", r);
      }
      total += tokens[r];
    }
    if (total <= 0) return fail(DDP_EINVAL, "total token count must be > 0");
    // binary32 nearest to the integer total (the conversion rounds to
    // nearest even); exact up to 2^24.
    out->divisor = static_cast<float>(total);
    divisor = out->divisor;
  } else {
    return fail(DDP_EINVAL, "unknown averaging mode %d", avg_mode);
  }
  const float d = static_cast<float>(divisor);
  out->divisor = d;
  out->recip = 1.0f;
  int e = 0;
  const float m = std::frexp(d, &e);  // d = m * 2^e, m in [0.5, 1)
  if (d == 1.0f) {
    out->mode = kNone;
  } else if (m == 0.5f && e - 1 <= 126) {
    out->mode = kScale;  // d = 2^(e-1): its reciprocal is exact
    out->recip = std::ldexp(1.0f, -(e - 1));
  } else {
    out->mode = kDivide;
  }
  return DDP_OK;
}

ddp_status validate_allreduce(void *const *bufs, int32_t p, int64_t n, int32_t dtype,
                              int32_t avg_mode, const int64_t *tokens, Divide *div,
                              const char *what) {
  ddp_status s = check_p(p, what);
  if (s != DDP_OK) return s;
  if (n < 0) return fail(DDP_EINVAL, "%s: n=%lld is negative", what, (long long)n);
  const int eb = elem_bytes_of(dtype);
  if (eb == 0) return fail(DDP_EINVAL, "%s: unknown dtype %d", what, dtype);
  s = make_divide(avg_mode, p, tokens, div);
  if (s != DDP_OK) return s;
  return check_rank_buffers(what, bufs, p, n * eb);
}

ddp_status check_workspace(const char *what, const void *workspace, size_t workspace_bytes,
                           size_t need, const void *const *bufs, int32_t p,
                           int64_t buf_bytes) {
  if (need == 0) return DDP_OK;
  if (workspace == nullptr || workspace_bytes < need) {
    return fail(DDP_EWORKSPACE, "%s: needs %zu workspace bytes, got %zu", what, need,
                workspace == nullptr ? size_t(0) : workspace_bytes);
  }
  if (reinterpret_cast<uintptr_t>(workspace) % kVecBytes != 0) {
    return fail(DDP_EALIGN, "%s: workspace is not 16-byte aligned", what);
  }
  for (int32_t r = 0; r < p; ++r) {
    if (ranges_overlap(workspace, int64_t(need), bufs[r], buf_bytes)) {
      return fail(DDP_EALIAS, "%s: workspace overlaps rank %d", what, r);
    }
  }
  return DDP_OK;
}

RankTable make_table(const void *const *bufs, int32_t p) {
  RankTable t;
  std::memset(&t, 0, sizeof t);
  for (int32_t r = 0; r < p; ++r) t.ptr[r] = const_cast<void *>(bufs[r]);
  return t;
}

size_t residency_lds(int32_t wgs) {
  if (wgs <= 0) return 0;
  constexpr int kMaxDevices = 64;
  // by device: LDS per CU and the most one workgroup may take (0 = not asked)
  static int32_t per_cu_of[kMaxDevices], per_wg_of[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return 0;
  }
  const bool cached = dev >= 0 && dev < kMaxDevices;
  int per_cu = cached ? __atomic_load_n(&per_cu_of[dev], __ATOMIC_RELAXED) : 0;
  int per_wg = cached ? __atomic_load_n(&per_wg_of[dev], __ATOMIC_RELAXED) : 0;
  if (per_cu == 0 || per_wg == 0) {
    if (hipDeviceGetAttribute(&per_cu, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor,
                              dev) != hipSuccess ||
        hipDeviceGetAttribute(&per_wg, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) !=
            hipSuccess ||
        per_cu <= 0 || per_wg <= 0) {
      (void)hipGetLastError();
      return 0;
    }
    if (cached) {
      __atomic_store_n(&per_wg_of[dev], per_wg, __ATOMIC_RELAXED);
      __atomic_store_n(&per_cu_of[dev], per_cu, __ATOMIC_RELAXED);
    }
  }
  // a bound below LDS-per-CU / max-per-workgroup cannot be reached this way
  const size_t bytes = static_cast<size_t>(per_cu / wgs) / 512 * 512;
  return bytes <= static_cast<size_t>(per_wg) ? bytes : static_cast<size_t>(per_wg) / 512 * 512;
}

#ifndef DDPSIM_RESIDENCY_SCALE
// With the bound of 8 ranks kept at 2 ranks, a 2-rank fused all-reduce
// and reduce-scatter of 1 GiB ran at 0.61 and 0.58 of 8 TB/s; scaled, 0.86
// and 0.85 (8 ranks and more: unchanged).
#define DDPSIM_RESIDENCY_SCALE 1
#endif
int32_t fold_residency(int32_t wgs, int32_t p) {
  if (wgs <= 0 || p >= 8 || p < 1 || !DDPSIM_RESIDENCY_SCALE) return wgs;
  return (wgs * 8 + p - 1) / p;
}

int32_t fanout_waves(int32_t dests) {
  int32_t w = 1;
  while (w < kMaxFanoutWaves && w * DDPSIM_FANOUT_DESTS_PER_WAVE < dests) w *= 2;
  return w;
}

}  // namespace ddpsim

using namespace ddpsim;

extern "C" const char *ddp_strerror(ddp_status s) {
  switch (s) {
    case DDP_OK: return "success";
    case DDP_EINVAL: return "invalid argument";
    case DDP_ERANGE: return "argument out of range";
    case DDP_EALIGN: return "buffer not 16-byte aligned";
    case DDP_EALIAS: return "buffers overlap";
    case DDP_ENOTDIVISIBLE: return "element count not divisible by the number of ranks";
    case DDP_ENOTREADY: return "plan has no device table";
    case DDP_EWORKSPACE: return "workspace missing or too small";
    case DDP_EHIP: return "HIP runtime error";
  }
  return "unknown status";
}

extern "C" const char *ddp_last_error(void) { return g_last_error; }

extern "C" const char *ddp_version(void) { return "ddpsim 0.1 (gfx950)"; }

extern "C" ddp_status ddp_time_next_call(hipEvent_t start, hipEvent_t stop) {
  clear_error();
  if ((start == nullptr) != (stop == nullptr)) {
    return fail(DDP_EINVAL, "ddp_time_next_call: pass both events or neither");
  }
  g_timer_start = start;
  g_timer_stop = stop;
  return DDP_OK;
}
