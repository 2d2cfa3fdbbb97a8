// bucket_allreduce.hip -- the bucket's all-reduce done in place on the
// per-parameter gradients: the same bits as ddp_flatten, then
// ring_allreduce_sim on the flat buffers, then ddp_unflatten, in one pass
// over HBM.
//
// The reducer copies every gradient into its slot of the bucket's flat
// buffer, all-reduces the buffer and copies the result back ("PyTorch DDP
// Deep Dive", Part 2 "Step 2: backward" item 1 and "Step 3:
// finalize_backward"). The ring's chunk geometry lives in the bucket's flat
// index space ("Collective Ops From Scratch", "Ring allreduce in two
// passes"). Nothing in that arithmetic needs the flat copy to exist: element
// j of parameter i is element offset_i + j of the bucket, and its ring chunk
// is (offset_i + j) / C. So a workgroup takes a tile of one parameter, folds
// every element across the p ranks' gradients of that parameter in ring
// order starting at the element's chunk, and writes the result back to all
// p ranks. HBM traffic 2 p n eb per bucket instead of 6 p n eb.
//
// A tile inside one chunk folds with one rank order for the whole wave. A
// tile that crosses chunk boundaries (small parameters, small chunks) folds
// per lane: each lane loads the ranks in the order of the chunk of its
// vector's first element, and an element whose chunk starts d ranks later
// skips the first d loads and adds them at the end, which is its own ring
// order. Tiles are therefore whole parameters cut into 64-vector runs, with
// no lanes left idle at chunk ends.
#include <algorithm>

#include "fold.hpp"
#include "internal.hpp"

namespace ddpsim {
int32_t plan_num_buckets(const ddp_plan *plan);
const int32_t *plan_tile_map(const ddp_plan *plan, int64_t *stride);
bool plan_segment_info(const ddp_plan *plan, int32_t b, int32_t *first, int32_t *count,
                       int32_t *tiles, int32_t *tile_first, int64_t *elems,
                       const void **table, int32_t *seg_p, int32_t *n_params,
                       int32_t *elem_bytes);

namespace {

// Element j of a parameter at bucket offset `off` is in ring chunk
// (off + j) / C; j may run past the parameter by a few elements (a clamped
// lane), which only moves the chunk of results that are never stored.
__device__ __forceinline__ int32_t chunk_of(int64_t off, int64_t j, int64_t C) {
  return static_cast<int32_t>((off + j) / C);
}

// The fold of one lane's vectors when the ranks' order differs between
// lanes: lane-held rank addresses (lane r holds rank r's, moved back by the
// alignment shift) are fetched per lane with a cross-lane read. For vector
// u, c0 is the chunk of its first element and dist[e] how many chunks later
// element e's chunk starts (0..V-1; it is below p because every chunk index
// is). Loads run in the order c0, c0+1, ...; element e adds load t only from
// t = dist[e] on, then loads 0..dist[e]-1 after the last one, so it sums
// ranks c0+dist[e], ..., c0+dist[e]+p-1 (mod p) left to right: its own
// ring order.
template <typename Tr, int RB, bool kNT>
__device__ __forceinline__ void fold_vector_per_lane(uint64_t mine, int32_t p, int32_t c0,
                                                     const int32_t (&dist)[Tr::kVec],
                                                     int64_t vi, bool ok,
                                                     float (&acc)[Tr::kVec]) {
  constexpr int V = Tr::kVec;
  static_assert(RB >= V - 1, "the first batch must hold the loads added last");
#pragma unroll
  for (int e = 0; e < V; ++e) acc[e] = -0.0f;
  uint4 keep[V > 1 ? V - 1 : 1];
  const uint32_t lo = static_cast<uint32_t>(mine);
  const uint32_t hi = static_cast<uint32_t>(mine >> 32);
  for (int32_t s0 = 0; s0 < p; s0 += RB) {
    uint4 x[RB];
#pragma unroll
    for (int j = 0; j < RB; ++j) {
      const bool live = s0 + j < p;  // wave-uniform
      x[j] = make_uint4(0, 0, 0, 0);
      if (live) {
        const int32_t r = ring_rank(c0, s0 + j, p);
        // every lane takes part in the cross-lane reads (no divergence here)
        const uint32_t alo = static_cast<uint32_t>(__shfl(static_cast<int>(lo), r, 64));
        const uint32_t ahi = static_cast<uint32_t>(__shfl(static_cast<int>(hi), r, 64));
        const void *src =
            reinterpret_cast<const void *>((static_cast<uint64_t>(ahi) << 32) | alo);
        if (ok) x[j] = load_vec<kNT>(src, vi);
      }
    }
    if (s0 == 0) {
#pragma unroll
      for (int j = 0; j < V - 1; ++j) keep[j] = x[j];
    }
#pragma unroll
    for (int j = 0; j < RB; ++j) {
      const int32_t t = s0 + j;
      if (t < p) {
        float w[V];
        Tr::widen(x[j], w);
#pragma unroll
        for (int e = 0; e < V; ++e) {
          if (t >= dist[e]) acc[e] = acc[e] + w[e];
        }
      }
    }
  }
#pragma unroll
  for (int j = 0; j < V - 1; ++j) {
    if (j < p) {
      float w[V];
      Tr::widen(keep[j], w);
#pragma unroll
      for (int e = 0; e < V; ++e) {
        if (j < dist[e]) acc[e] = acc[e] + w[e];
      }
    }
  }
}

// One tile of the plan's numbering; the tile map names the parameter
// descriptor (index into seg) each tile belongs to.
template <typename Tr, int VPT, int RB, bool kNT>
__device__ __forceinline__ void bucket_tile(const SegDesc *__restrict__ seg,
                                            const int32_t *__restrict__ tile_seg,
                                            int64_t map_stride, int32_t tile, int32_t n_params,
                                            const void *const *__restrict__ grads, int32_t p,
                                            const Divide &div) {
  constexpr int V = Tr::kVec;
  constexpr int64_t kElemBytes = sizeof(typename Tr::elem);
  const SegDesc d = seg[tile_seg[tile_map_index(tile, map_stride)]];
  const int32_t t = tile - d.tile_begin;
  const int tid = static_cast<int>(threadIdx.x);
  constexpr int kThr = kBucketThreads;
  constexpr int64_t kTile = int64_t(kThr) * VPT * V;

  // The vector path needs every rank's copy of this parameter to sit at the
  // same offset from a 16-byte boundary.
  // lane r loads rank r's address (p <= 64 = the wave size)
  const int my_lane = tid & 63;
  const uint64_t mine =
      my_lane < p
          ? reinterpret_cast<uint64_t>(grads[static_cast<int64_t>(my_lane) * n_params + d.param])
          : 0;
  const uintptr_t phase =
      __builtin_amdgcn_readlane(static_cast<uint32_t>(mine), 0) % static_cast<uint32_t>(kVecBytes);
  const bool same =
      phase % kElemBytes == 0 && __all(my_lane >= p || mine % kVecBytes == phase);

  if (!same) {
    const GradPtrs at{grads, n_params, d.param, 0};
    const int64_t j0 = static_cast<int64_t>(t) * kTile;
    const int64_t j1 = std::min(j0 + kTile, d.len);
    for (int64_t j = j0 + tid; j < j1; j += kThr) {
      const float y = apply_divide(fold_scalar<Tr>(at, p, chunk_of(d.offset, j, d.chunk), j), div);
      for (int32_t r = 0; r < p; ++r) Tr::store1(at(r), j, y);
    }
    return;
  }

  // Shifted coordinates: index J = j + m addresses element j of the
  // parameter from a base moved back by m elements, which is 16-byte
  // aligned for every rank.
  const int64_t m = static_cast<int64_t>(phase) / kElemBytes;
  const GradPtrs at{grads, n_params, d.param, m * kElemBytes};
  const ChunkSpan k = make_span(m, d.len + m, V);

  if (t == 0 && tid >= kThr - 2 * (V - 1)) {
    const int lane = tid - (kThr - 2 * (V - 1));
    const bool head = lane < V - 1;
    const int64_t J = head ? k.s + lane : k.tail_begin + (lane - (V - 1));
    if (J < (head ? k.head_end : k.e)) {
      const float y =
          apply_divide(fold_scalar<Tr>(at, p, chunk_of(d.offset, J - m, d.chunk), J), div);
      for (int32_t r = 0; r < p; ++r) Tr::store1(at(r), J, y);
    }
  }

  const int64_t nv = (k.ve - k.vs) / V;
  const int64_t base = static_cast<int64_t>(t) * (kThr * VPT);
  if (base >= nv) return;
  int64_t vi[VPT];
  bool ok[VPT];
#pragma unroll
  for (int u = 0; u < VPT; ++u) {
    const int64_t jj = base + u * kThr + tid;
    ok[u] = jj < nv;
    vi[u] = k.vs / V + jj;
  }
  const uint64_t shifted = mine - static_cast<uint64_t>(m * kElemBytes);
  const LanePtrs lat{shifted};
  // chunks of the tile's first and last element (wave-uniform)
  const int64_t last_v = k.vs / V + std::min(base + int64_t(kThr) * VPT, nv) - 1;
  const int32_t c_first = chunk_of(d.offset, k.vs + base * V - m, d.chunk);
  const int32_t c_last = chunk_of(d.offset, last_v * V + V - 1 - m, d.chunk);
  float acc[VPT][V];
  if (c_first == c_last) {
    fold_vectors<Tr, VPT, RB, kNT>(lat, p, c_first, vi, ok, acc);
  } else {
#pragma unroll
    for (int u = 0; u < VPT; ++u) {
      // a lane past the body computes with the last vector (never stored)
      const int64_t v = ok[u] ? vi[u] : last_v;
      const int64_t j0 = v * V - m;
      const int32_t c0 = chunk_of(d.offset, j0, d.chunk);
      int32_t dist[V];
      int64_t next = (static_cast<int64_t>(c0) + 1) * d.chunk - d.offset;  // next chunk's first j
      int32_t dd = 0;
#pragma unroll
      for (int e = 0; e < V; ++e) {
        while (j0 + e >= next) {
          ++dd;
          next += d.chunk;
        }
        dist[e] = dd;
      }
      fold_vector_per_lane<Tr, RB, kNT>(shifted, p, c0, dist, vi[u], ok[u], acc[u]);
    }
  }
  uint4 y[VPT];
#pragma unroll
  for (int u = 0; u < VPT; ++u) {
#pragma unroll
    for (int e = 0; e < V; ++e) acc[u][e] = apply_divide(acc[u][e], div);
    y[u] = Tr::narrow(acc[u]);
  }
  const int32_t rot = store_rotation(p, tile);
  for (int32_t r = 0; r < p; ++r) {
    void *dst = lat(ring_rank(rot, r, p));
#pragma unroll
    for (int u = 0; u < VPT; ++u) {
      if (ok[u]) store_vec<kNT>(dst, vi[u], y[u]);
    }
  }
}

// Workgroup w handles tiles tile_base + w, + gridDim.x, ... of the n_tiles
// of a run of buckets: one tile each when the grid covers them all (the
// default), several when the caller capped the number of workgroups so the
// all-reduce leaves compute units to kernels running beside it.
template <typename Tr, int VPT, int RB, bool kNT>
__global__ __launch_bounds__(kBucketThreads) void bucket_allreduce_kernel(
    const SegDesc *__restrict__ seg, const int32_t *__restrict__ tile_seg, int64_t map_stride,
    int32_t tile_base, int32_t n_tiles, int32_t n_params,
    const void *const *__restrict__ grads, int32_t p, Divide div) {
  for (int32_t w = static_cast<int32_t>(blockIdx.x); w < n_tiles;
       w += static_cast<int32_t>(gridDim.x)) {
    bucket_tile<Tr, VPT, RB, kNT>(seg, tile_seg, map_stride, tile_base + w, n_params, grads, p,
                                  div);
  }
}

}  // namespace
}  // namespace ddpsim

using namespace ddpsim;

namespace ddpsim {

ddp_status allreduce_buckets(const ddp_plan *plan, int32_t first_bucket, int32_t n_buckets,
                             int32_t p, void *const *d_grad_ptrs, int32_t dtype,
                             int32_t avg_mode, const int64_t *tokens, hipStream_t stream,
                             ddp_comm_stats *stats, int32_t max_workgroups) {
  clear_error();
  CallTimer timer = CallTimer::take();
  const char *what = "ddp_allreduce_buckets";
  if (plan == nullptr) return fail(DDP_EINVAL, "%s: plan is NULL", what);
  const int32_t nbk = plan_num_buckets(plan);
  if (n_buckets < 1 || first_bucket < 0 || first_bucket >= nbk ||
      n_buckets > nbk - first_bucket) {
    return fail(DDP_ERANGE, "%s: buckets [%d, %d) outside [0, %d)", what, first_bucket,
                first_bucket + n_buckets, nbk);
  }
  ddp_status s = check_p(p, what);
  if (s != DDP_OK) return s;
  int32_t seg0 = 0, nseg = 0, tiles = 0, tile0 = 0, seg_p = 0, n_params = 0, eb_plan = 0;
  int64_t elems = 0;
  const void *table = nullptr;
  int64_t C_sum = 0;
  for (int32_t b = first_bucket; b < first_bucket + n_buckets; ++b) {
    int32_t f, c, t, tf;
    int64_t e;
    plan_segment_info(plan, b, &f, &c, &t, &tf, &e, &table, &seg_p, &n_params, &eb_plan);
    if (seg_p != p) {
      return fail(DDP_ENOTREADY, "%s: call ddp_plan_upload_segments with p=%d first", what, p);
    }
    if (b == first_bucket) {
      seg0 = f;
      tile0 = tf;
    }
    nseg += c;
    tiles += t;
    elems += e;
    C_sum += e > 0 ? ceil_div(e, p) : 0;
  }
  const int eb = elem_bytes_of(dtype);
  if (eb == 0) return fail(DDP_EINVAL, "%s: unknown dtype %d", what, dtype);
  if (eb != eb_plan) {
    return fail(DDP_EINVAL, "%s: dtype has %d-byte elements, the plan %d", what, eb, eb_plan);
  }
  if (tiles > 0 && d_grad_ptrs == nullptr) {
    return fail(DDP_EINVAL, "%s: gradient pointer table is NULL", what);
  }
  Divide div;
  s = make_divide(avg_mode, p, tokens, &div);
  if (s != DDP_OK) return s;
  if (stats != nullptr) {
    // one ring all-reduce per bucket
    stats->steps = 2 * int64_t(p - 1) * n_buckets;
    stats->messages = 2 * int64_t(p) * (p - 1) * n_buckets;
    stats->bytes_sent_per_rank = 2 * int64_t(p - 1) * C_sum * 4;
    stats->bytes_recv_per_rank = stats->bytes_sent_per_rank;
    stats->total_bytes = 2 * int64_t(p) * (p - 1) * C_sum * 4;
    stats->hbm_bytes = 2 * int64_t(p) * elems * eb;
  }
  if (tiles == 0) return DDP_OK;
  (void)seg0;
  (void)nseg;
  const SegDesc *seg = static_cast<const SegDesc *>(table);
  int64_t map_stride = 0;
  const int32_t *tile_seg = plan_tile_map(plan, &map_stride);
  const void *const *grads = d_grad_ptrs;
  const int32_t blocks = max_workgroups > 0 ? std::min(tiles, max_workgroups) : tiles;
  const dim3 grid(static_cast<uint32_t>(blocks));
  // Each workgroup keeps 2p streams of 1 KiB in flight (p loads, p
  // stores); a CU full of them (32 one-wave workgroups) puts more streams on
  // every HBM channel than it keeps rows open. Bounding residency at 11 per
  // CU raised the GPT-2 p=8 launch from 5.76 to 6.05 TB/s and the Llama bf16
  // buckets by 3-4%; 6 per CU starved the channels (5.2).
  const size_t lds = residency_lds(fold_residency(DDPSIM_BUCKET_WGS_PER_CU, p));
  if (dtype == DDP_F32) {
    return launch_lds(bucket_allreduce_kernel<F32Traits, kBucketVpt, kBucketRb, kBucketNt>, grid,
                      dim3(kBucketThreads), lds, stream, timer, true,
                      "bucket_allreduce_kernel launch", seg, tile_seg, map_stride, tile0, tiles, n_params,
                      grads, p, div);
  }
  return launch_lds(bucket_allreduce_kernel<BF16Traits, kBucketVpt, kBucketRb, kBucketNt>, grid,
                    dim3(kBucketThreads), lds, stream, timer, true,
                    "bucket_allreduce_kernel launch", seg, tile_seg, map_stride, tile0, tiles, n_params, grads,
                    p, div);
}

}  // namespace ddpsim

extern "C" ddp_status ddp_allreduce_buckets(const ddp_plan *plan, int32_t first_bucket,
                                            int32_t n_buckets, int32_t p,
                                            void *const *d_grad_ptrs, int32_t dtype,
                                            int32_t avg_mode, const int64_t *tokens,
                                            hipStream_t stream, ddp_comm_stats *stats) {
  return allreduce_buckets(plan, first_bucket, n_buckets, p, d_grad_ptrs, dtype, avg_mode,
                           tokens, stream, stats, DDPSIM_BUCKET_MAX_WORKGROUPS);
}

extern "C" ddp_status ddp_allreduce_bucket(const ddp_plan *plan, int32_t bucket, int32_t p,
                                           void *const *d_grad_ptrs, int32_t dtype,
                                           int32_t avg_mode, const int64_t *tokens,
                                           hipStream_t stream, ddp_comm_stats *stats) {
  if (plan != nullptr && (bucket < 0 || bucket >= plan_num_buckets(plan))) {
    clear_error();
    CallTimer::take();
    return fail(DDP_ERANGE, "ddp_allreduce_bucket: bucket %d out of range", bucket);
  }
  return ddp_allreduce_buckets(plan, bucket, 1, p, d_grad_ptrs, dtype, avg_mode, tokens,
                               stream, stats);
}
