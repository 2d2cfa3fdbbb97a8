// fold.hpp -- the ring-order fold, shared by the fused all-reduce, the
// in-place bucket all-reduce and the fused reduce-scatter kernels.
//
// The ring's reduce-scatter carries chunk c from rank c to rank c+1, c+2,
// ... and each hop adds that rank's own, still untouched value ("Data
// parallelism", section "Ring all-reduce, derived"). So the finished sum of
// any element of chunk c is
//     x[first] + x[first+1] + ... + x[first+p-1]      (ranks mod p)
// accumulated left to right in fp32, with first = c for the all-reduce and
// first = c+1 for the pre-rotated reduce-scatter. The kernels below reproduce
// that order exactly while keeping every load of a batch in flight at once:
// loads do not depend on each other, only the additions are ordered.
//
// The accumulator starts at -0.0f: -0 + x == x for every x (including +0
// and -0), so adding all p values to it gives the same bits as starting
// from x[first].
#pragma once

#include "internal.hpp"

namespace ddpsim {

// Where a kernel finds rank r's base address: the kernel-argument table...
struct TablePtrs {
  const RankTable &tab;
  __device__ __forceinline__ void *operator()(int32_t r) const { return tab.ptr[r]; }
};

// ...or a device array of p * n_params gradient addresses (rank-major), for
// one parameter, moved back by `shift` bytes so that the vector grid of all
// ranks starts on a 16-byte boundary.
struct GradPtrs {
  const void *const *tab;
  int32_t n_params;
  int32_t param;
  int64_t shift;
  __device__ __forceinline__ void *operator()(int32_t r) const {
    return const_cast<char *>(static_cast<const char *>(
               tab[static_cast<int64_t>(r) * n_params + param])) - shift;
  }
};

// ...or one address per lane: lane r of the wave holds rank r's base
// address (moved back by the same shift), and a wave-uniform rank index
// reads it with readlane. The p addresses then cost one vector load per
// workgroup instead of p scalar loads. Only for wave-uniform rank indices in
// code every lane runs (the fold's and the stores' rank loops).
struct LanePtrs {
  uint64_t mine;
  __device__ __forceinline__ void *operator()(int32_t r) const {
    const uint32_t lo = __builtin_amdgcn_readlane(static_cast<uint32_t>(mine), r);
    const uint32_t hi = __builtin_amdgcn_readlane(static_cast<uint32_t>(mine >> 32), r);
    return reinterpret_cast<void *>((static_cast<uint64_t>(hi) << 32) | lo);
  }
};

// Fold VPT 16-byte vectors (vector indices vi[u], valid where ok[u]) over
// the p ranks in ring order starting at `first`. RB rank loads are issued
// before their additions; kNT makes them non-temporal.
template <typename Tr, int VPT, int RB, bool kNT, typename Ptrs>
__device__ __forceinline__ void fold_vectors(const Ptrs &ptr_of, int32_t p,
                                             int32_t first,
                                             const int64_t (&vi)[VPT],
                                             const bool (&ok)[VPT],
                                             float (&acc)[VPT][Tr::kVec]) {
#pragma unroll
  for (int u = 0; u < VPT; ++u) {
#pragma unroll
    for (int e = 0; e < Tr::kVec; ++e) acc[u][e] = -0.0f;
  }
  for (int32_t s0 = 0; s0 < p; s0 += RB) {
    uint4 x[RB][VPT];
#pragma unroll
    for (int j = 0; j < RB; ++j) {
      const bool live = s0 + j < p;
      const void *src = ptr_of(live ? ring_rank(first, s0 + j, p) : 0);
#pragma unroll
      for (int u = 0; u < VPT; ++u) {
        x[j][u] = (live && ok[u]) ? load_vec<kNT>(src, vi[u]) : make_uint4(0, 0, 0, 0);
      }
    }
#pragma unroll
    for (int j = 0; j < RB; ++j) {
      if (s0 + j < p) {
#pragma unroll
        for (int u = 0; u < VPT; ++u) {
          float w[Tr::kVec];
          Tr::widen(x[j][u], w);
#pragma unroll
          for (int e = 0; e < Tr::kVec; ++e) acc[u][e] = acc[u][e] + w[e];
        }
      }
    }
  }
}

// The same fold for one element. Loads go out in batches of 32 ranks
// before their additions, so p = 64 costs two memory latencies, not 64.
template <typename Tr, typename Ptrs>
__device__ __forceinline__ float fold_scalar(const Ptrs &ptr_of, int32_t p,
                                             int32_t first, int64_t i) {
  constexpr int kBatch = 32;
  float acc = -0.0f;
  for (int32_t s0 = 0; s0 < p; s0 += kBatch) {
    float x[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      x[j] = s0 + j < p ? Tr::load1(ptr_of(ring_rank(first, s0 + j, p)), i) : 0.0f;
    }
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      if (s0 + j < p) acc = acc + x[j];
    }
  }
  return acc;
}

}  // namespace ddpsim
