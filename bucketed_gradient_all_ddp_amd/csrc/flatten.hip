// flatten.hip -- copy gradients into a bucket's flat buffer and back
// ("PyTorch DDP Deep Dive", Part 2 "Step 2: backward", the reducer's copy of
// each gradient into its slice of the bucket, with the optional pre-divide;
// "Step 3: finalize_backward", the copy back into each .grad).
//
// One launch handles one bucket for all p ranks: grid (spans, p). Each
// parameter of the bucket is cut into tiles of kFlattenTile elements, each
// tile into spans of one 16-byte vector per lane of a workgroup, and a
// workgroup finds its parameter through the tile map that follows the
// descriptors in the plan's device table (one scalar load). A tile whose source and destination are both
// 16-byte aligned moves 16-byte vectors; any other tile moves elements.
#include <cmath>

#include "internal.hpp"

namespace ddpsim {
bool plan_bucket_info(const ddp_plan *plan, int32_t b, int32_t *first,
                      int32_t *count, int32_t *tiles, int64_t *elems,
                      const void **table, const int32_t **tile_map, int32_t *n_params,
                      int32_t *elem_bytes, bool *uploaded);

namespace {

#ifndef DDPSIM_FLAT_THREADS
#define DDPSIM_FLAT_THREADS 64  // threads per workgroup, one 16-byte vector each
#endif
#ifndef DDPSIM_FLAT_NT
// bit 0: non-temporal loads; bit 1: non-temporal stores. Loads only: the
// flat bucket ddp_flatten writes is read next by the all-reduce, which finds
// it in the Infinity Cache when the stores are ordinary.
#define DDPSIM_FLAT_NT 1
#endif
constexpr int kFlatThreads = DDPSIM_FLAT_THREADS;
constexpr bool kFlatNtLoad = (DDPSIM_FLAT_NT & 1) != 0;
constexpr bool kFlatNtStore = (DDPSIM_FLAT_NT & 2) != 0;

// Workgroup (w, r) copies the w % S-th span of kFlatThreads vectors of plan
// tile w / S (S = spans per tile) for rank r: many small workgroups with one
// vector per lane stream best on gfx950.
template <typename Tr, bool kToFlat>
__global__ __launch_bounds__(kFlatThreads) void flatten_kernel(
    const ParamDesc *__restrict__ desc, const int32_t *__restrict__ tile_map, int32_t n_params,
    const void *const *__restrict__ grad_ptrs, RankTable flat, Divide div) {
  constexpr int V = Tr::kVec;
  constexpr int kSpan = kFlatThreads * V;  // elements per workgroup
  constexpr int kSubs = kFlattenTile / kSpan;
  static_assert(kSubs >= 1 && kSubs * kSpan == kFlattenTile, "spans must tile a plan tile");
  using E = typename Tr::elem;
  const int32_t tile = static_cast<int32_t>(blockIdx.x) / kSubs;
  const int32_t sub = static_cast<int32_t>(blockIdx.x) - tile * kSubs;
  const int32_t r = static_cast<int32_t>(blockIdx.y);
  const ParamDesc d = desc[tile_map[tile]];
  const int64_t start = static_cast<int64_t>(tile - d.tile_begin) * kFlattenTile +
                        static_cast<int64_t>(sub) * kSpan;
  const int64_t left = d.numel - start;
  if (left <= 0) return;
  const int64_t cnt = left < kSpan ? left : kSpan;
  E *grad = static_cast<E *>(const_cast<void *>(
                grad_ptrs[static_cast<int64_t>(r) * n_params + d.param])) + start;
  E *bucket = static_cast<E *>(flat.ptr[r]) + d.bucket_offset + start;
  const E *src = kToFlat ? grad : bucket;
  E *dst = kToFlat ? bucket : grad;
  const bool scale = kToFlat && div.mode != kNone;
  const int tid = static_cast<int>(threadIdx.x);

  const bool aligned = ((reinterpret_cast<uintptr_t>(src) |
                         reinterpret_cast<uintptr_t>(dst)) % kVecBytes) == 0;
  int64_t done = 0;
  if (aligned) {
    const int64_t nv = cnt / V;
    if (tid < nv) {
      uint4 x = load_vec<kFlatNtLoad>(src, tid);
      if (scale) {
        float f[V];
        Tr::widen(x, f);
#pragma unroll
        for (int e = 0; e < V; ++e) f[e] = apply_divide(f[e], div);
        x = Tr::narrow(f);
      }
      store_vec<kFlatNtStore>(dst, tid, x);
    }
    done = nv * V;
  }
  for (int64_t i = done + tid; i < cnt; i += kFlatThreads) {
    if (scale) {
      Tr::store1(dst, i, apply_divide(Tr::load1(src, i), div));
    } else {
      global_ptr<E>(dst)[i] = global_ptr<E>(src)[i];
    }
  }
}

ddp_status run(const ddp_plan *plan, int32_t bucket, int32_t p,
               const void *const *d_grad_ptrs, const void *const *bucket_bufs,
               int32_t dtype, float prescale, bool to_flat, hipStream_t stream,
               const char *what) {
  clear_error();
  CallTimer timer = CallTimer::take();
  int32_t first, count, tiles, n_params, eb_plan;
  int64_t elems;
  const void *table;
  const int32_t *tile_map;
  bool uploaded;
  if (plan == nullptr) return fail(DDP_EINVAL, "%s: plan is NULL", what);
  if (!plan_bucket_info(plan, bucket, &first, &count, &tiles, &elems, &table, &tile_map,
                        &n_params, &eb_plan, &uploaded)) {
    return fail(DDP_ERANGE, "%s: bucket %d out of range", what, bucket);
  }
  if (!uploaded) return fail(DDP_ENOTREADY, "%s: call ddp_plan_upload first", what);
  ddp_status s = check_p(p, what);
  if (s != DDP_OK) return s;
  const int eb = elem_bytes_of(dtype);
  if (eb == 0) return fail(DDP_EINVAL, "%s: unknown dtype %d", what, dtype);
  if (eb != eb_plan) {
    return fail(DDP_EINVAL, "%s: dtype has %d-byte elements, the plan %d", what, eb, eb_plan);
  }
  if (!(prescale > 0.0f) || prescale > 3.0e38f) {
    return fail(DDP_EINVAL, "%s: prescale divisor must be finite and > 0", what);
  }
  if (tiles > 0 && d_grad_ptrs == nullptr) {
    return fail(DDP_EINVAL, "%s: gradient pointer table is NULL", what);
  }
  s = check_rank_buffers(what, bucket_bufs, p, elems * eb);
  if (s != DDP_OK) return s;
  if (tiles == 0) return DDP_OK;
  Divide div{kNone, 1.0f, 1.0f};
  if (prescale != 1.0f) {
    int e = 0;
    const float m = std::frexp(prescale, &e);
    if (m == 0.5f && e - 1 <= 126 && e - 1 >= -126) {
      div = Divide{kScale, prescale, std::ldexp(1.0f, -(e - 1))};
    } else {
      div = Divide{kDivide, prescale, 1.0f};
    }
  }
  const ParamDesc *desc = static_cast<const ParamDesc *>(table) + first;
  const RankTable tab = make_table(bucket_bufs, p);
  const int vec = dtype == DDP_F32 ? 4 : 8;
  const int64_t blocks = int64_t(tiles) * (kFlattenTile / (kFlatThreads * vec));
  if (blocks > INT32_MAX) return fail(DDP_EINVAL, "%s: bucket too large", what);
  const dim3 grid(static_cast<uint32_t>(blocks), static_cast<uint32_t>(p));
  const char *kname = "flatten_kernel launch";
  if (dtype == DDP_F32) {
    if (to_flat) {
      return launch(flatten_kernel<F32Traits, true>, grid, dim3(kFlatThreads), stream, timer, true,
                    kname, desc, tile_map, n_params, d_grad_ptrs, tab, div);
    }
    return launch(flatten_kernel<F32Traits, false>, grid, dim3(kFlatThreads), stream, timer, true,
                  kname, desc, tile_map, n_params, d_grad_ptrs, tab, div);
  }
  if (to_flat) {
    return launch(flatten_kernel<BF16Traits, true>, grid, dim3(kFlatThreads), stream, timer, true,
                  kname, desc, tile_map, n_params, d_grad_ptrs, tab, div);
  }
  return launch(flatten_kernel<BF16Traits, false>, grid, dim3(kFlatThreads), stream, timer, true,
                kname, desc, tile_map, n_params, d_grad_ptrs, tab, div);
}

}  // namespace
}  // namespace ddpsim

using namespace ddpsim;

extern "C" ddp_status ddp_flatten(const ddp_plan *plan, int32_t bucket, int32_t p,
                                  const void *const *d_grad_ptrs, void *const *bucket_bufs,
                                  int32_t dtype, float prescale_divisor,
                                  hipStream_t stream) {
  return run(plan, bucket, p, d_grad_ptrs, reinterpret_cast<const void *const *>(bucket_bufs),
             dtype, prescale_divisor, true, stream, "ddp_flatten");
}

extern "C" ddp_status ddp_unflatten(const ddp_plan *plan, int32_t bucket, int32_t p,
                                    const void *const *bucket_bufs, void *const *d_grad_ptrs,
                                    int32_t dtype, hipStream_t stream) {
  return run(plan, bucket, p, reinterpret_cast<const void *const *>(d_grad_ptrs), bucket_bufs,
             dtype, 1.0f, false, stream, "ddp_unflatten");
}
