// workspace.hpp -- fp32 workspace rows for the step-by-step all-reduce
// schedules on bf16 buffers: partial sums travel and accumulate in fp32, so
// bf16 rank buffers are widened into fp32 rows before the first step and
// rounded back once after the last.
#pragma once

#include "internal.hpp"

namespace ddpsim {

// fp32 elements between workspace rows: n rounded up to 256 bytes.
inline int64_t workspace_stride_elems(int64_t n) { return ceil_div(n * 4, 256) * 256 / 4; }

#if defined(__HIPCC__)
// bf16 rank buffers <-> fp32 workspace rows (row r at ws + r * stride).
template <bool kToWorkspace>
__global__ __launch_bounds__(kThreads) void bf16_workspace_kernel(
    RankTable bufs, float *ws, int64_t ws_stride, int64_t n,
    int32_t tiles_per_rank) {
  constexpr int kElems = 8;  // one 16-byte bf16 vector, two fp32 vectors
  const int32_t r = static_cast<int32_t>(blockIdx.x) / tiles_per_rank;
  const int32_t t = static_cast<int32_t>(blockIdx.x) - r * tiles_per_rank;
  uint16_t *b = static_cast<uint16_t *>(bufs.ptr[r]);
  float *w = ws + r * ws_stride;
  const int64_t v = static_cast<int64_t>(t) * kThreads + threadIdx.x;
  const int64_t i0 = v * kElems;
  if (i0 >= n) return;
  if (i0 + kElems <= n) {
    if (kToWorkspace) {
      float f[8];
      BF16Traits::widen(load_vec(b, v), f);
      store_vec<false>(w, 2 * v, make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]),
                                            __float_as_uint(f[2]), __float_as_uint(f[3])));
      store_vec<false>(w, 2 * v + 1, make_uint4(__float_as_uint(f[4]), __float_as_uint(f[5]),
                                                __float_as_uint(f[6]), __float_as_uint(f[7])));
    } else {
      float f[8];
      float lo[4], hi[4];
      F32Traits::widen(load_vec(w, 2 * v), lo);
      F32Traits::widen(load_vec(w, 2 * v + 1), hi);
      for (int e = 0; e < 4; ++e) {
        f[e] = lo[e];
        f[e + 4] = hi[e];
      }
      store_vec<false>(b, v, BF16Traits::narrow(f));
    }
  } else {
    for (int64_t i = i0; i < n; ++i) {
      if (kToWorkspace) {
        w[i] = BF16Traits::load1(b, i);
      } else {
        BF16Traits::store1(b, i, w[i]);
      }
    }
  }
}

#endif  // __HIPCC__

}  // namespace ddpsim
