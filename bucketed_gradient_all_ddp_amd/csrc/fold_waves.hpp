// fold_waves.hpp -- the ring-order fold of one tile with the tile's ranks
// split over the W waves of a workgroup, for the streaming kernels with many
// ranks (the fused all-reduce and the reduce-scatter).
//
// With one wave per tile a wave reads p ranks in batches of 8, and the
// batches of one tile follow each other; beyond 8 ranks more of the tile's
// loads can be in flight when W waves each take a contiguous share of the
// ring positions. The additions stay in ring order: wave 0 adds its values
// to -0.0, leaves the sum in LDS, and each later wave continues from the sum
// the wave before it left, so the result is bit for bit the left-to-right
// fold x[first] + x[first+1] + ... + x[first+p-1] of fold.hpp.
#pragma once

#include "fold.hpp"

namespace ddpsim {

// Fold the 16-byte vector vi (valid where ok) of one 64-lane tile over the p
// ranks in ring order from `first`. Wave `wave` of W holds ring positions
// [lo, hi) = [wave*p/W, (wave+1)*p/W), at most S of them; every wave of the
// workgroup must call this with the same tile (it contains W barriers), and
// every wave returns the finished sum in acc. slot is 64 * Tr::kVec floats
// of LDS that hold the sum after the call, so the kernels take one tile per
// workgroup.
template <typename Tr, int W, int S, typename Ptrs>
__device__ __forceinline__ void fold_tile_waves(const Ptrs &ptr_of, int32_t p, int32_t first,
                                                int32_t wave, int32_t lo, int32_t hi,
                                                int64_t vi, bool ok, float *slot,
                                                float (&acc)[Tr::kVec]) {
  constexpr int V = Tr::kVec;
  const int lane = static_cast<int>(threadIdx.x) & 63;
  // this wave's positions, every load in flight before the first add
  uint4 x[S];
#pragma unroll
  for (int j = 0; j < S; ++j) {
    const bool live = lo + j < hi;  // wave-uniform
    const void *src = ptr_of(live ? ring_rank(first, lo + j, p) : 0);
    x[j] = (live && ok) ? load_vec<true>(src, vi) : make_uint4(0, 0, 0, 0);
  }
  for (int32_t w = 0; w < W; ++w) {
    if (wave == w) {
#pragma unroll
      for (int e = 0; e < V; ++e) acc[e] = w == 0 ? -0.0f : slot[e * 64 + lane];
#pragma unroll
      for (int j = 0; j < S; ++j) {
        if (lo + j < hi) {
          float f[V];
          Tr::widen(x[j], f);
#pragma unroll
          for (int e = 0; e < V; ++e) acc[e] = acc[e] + f[e];
        }
      }
#pragma unroll
      for (int e = 0; e < V; ++e) slot[e * 64 + lane] = acc[e];
    }
    __syncthreads();
  }
#pragma unroll
  for (int e = 0; e < V; ++e) acc[e] = slot[e * 64 + lane];
}

}  // namespace ddpsim
