// coalesced.hip -- broadcast of many tensors from one rank, coalesced into
// capped buckets ("PyTorch DDP Deep Dive", Part 1: the init-time broadcast
// of parameters and buffers that makes the replicas identical; Part 2: the
// buffer broadcast before every forward, down to the coalesced broadcast
// with its 250 MiB buckets).
//
// On the pages each bucket is flattened at the root, broadcast as one flat
// buffer over the doubling tree, and unflattened on every rank. On one
// device the flat buffer is only a staging copy: each bucket is one launch
// that reads the root's tensors once and writes them straight into the other
// p - 1 ranks' tensors, so a bucket costs p bytes-per-element of device
// traffic instead of the 2 + 2p of flatten, fan-out and unflatten. Buckets
// run one after another on the stream. The tree's rounds and messages are
// kept in the accounting.
#include <algorithm>

#include "internal.hpp"

namespace ddpsim {
bool plan_bucket_info(const ddp_plan *plan, int32_t b, int32_t *first,
                      int32_t *count, int32_t *tiles, int64_t *elems,
                      const void **table, const int32_t **tile_map, int32_t *n_params,
                      int32_t *elem_bytes, bool *uploaded);
int32_t plan_num_buckets(const ddp_plan *plan);

namespace {

#ifndef DDPSIM_BCAST_NT
#define DDPSIM_BCAST_NT 0  // non-temporal loads of the root's tensors
#endif
constexpr bool kBcastNtLoad = DDPSIM_BCAST_NT != 0;
#ifndef DDPSIM_BCAST_NT_STORE_BYTES
// Buckets whose copies total more than this take non-temporal stores (the
// GPT-2 parameter sync, two buckets of 250 MiB to 7 ranks: +1%); smaller
// ones stay eligible for the Infinity Cache. Non-temporal loads as well
// lost 4%.
#define DDPSIM_BCAST_NT_STORE_BYTES (int64_t(256) << 20)
#endif
#ifndef DDPSIM_BCAST_THREADS
#define DDPSIM_BCAST_THREADS 64  // threads per workgroup, one 16-byte vector each
#endif
#ifndef DDPSIM_BCAST_VPT
#define DDPSIM_BCAST_VPT 1  // 16-byte vectors per lane (spans per workgroup)
#endif
#ifndef DDPSIM_BCAST_WGS_PER_CU
#define DDPSIM_BCAST_WGS_PER_CU 0  // workgroups resident per CU (0: no bound)
#endif
constexpr int kBcastThreads = DDPSIM_BCAST_THREADS;
constexpr int kBcastVpt = DDPSIM_BCAST_VPT;

template <int EB>
struct Unit;
template <>
struct Unit<1> { using type = uint8_t; };
template <>
struct Unit<2> { using type = uint16_t; };
template <>
struct Unit<4> { using type = uint32_t; };
template <>
struct Unit<8> { using type = uint64_t; };

#ifndef DDPSIM_BCAST_SPANS
// Consecutive spans per workgroup, each span's stores overlapping the next
// span's load. One is best: 2, 4 and 16 lost 5%, 5% and 12% on the GPT-2
// parameter sync (fewer, longer workgroups keep fewer loads in flight).
#define DDPSIM_BCAST_SPANS 1
#endif
constexpr int kBcastSpans = DDPSIM_BCAST_SPANS;

// Each plan tile of kFlattenTile elements of one tensor (named by the plan's
// tile map, as in flatten_kernel) is split into spans of one 16-byte vector
// per lane; a workgroup takes kBcastSpans consecutive spans of one tile. Its
// waves (fanout_waves of the p - 1 destinations) each load the root's span
// and store it to their own share of the other ranks; the next span's load
// is issued before this span's stores. 16-byte vectors when every
// rank's copy of the tensor is 16-byte aligned (spans start at multiples of
// 16 bytes from the tensor's base, so the base decides), elements of EB
// bytes otherwise.
// Spans per workgroup for EB-byte elements: at most the spans of one tile.
template <int EB>
constexpr int bcast_spans() {
  constexpr int per_tile = kFlattenTile * EB / (kBcastThreads * kBcastVpt * kVecBytes);
  return kBcastSpans < per_tile ? kBcastSpans : per_tile;
}

template <int EB, bool kNtStore>
__global__ __launch_bounds__(kBcastThreads * kMaxFanoutWaves) void coalesced_broadcast_kernel(
    const ParamDesc *__restrict__ desc, const int32_t *__restrict__ tile_map, int32_t n_params,
    const void *const *__restrict__ ptrs, int32_t p, int32_t root) {
  using U = typename Unit<EB>::type;
  constexpr int kSpans = bcast_spans<EB>();
  constexpr int kSpan = kBcastThreads * kBcastVpt * kVecBytes / EB;  // elements per span
  constexpr int kSubs = kFlattenTile / (kSpan * kSpans);             // workgroups per tile
  static_assert(kSubs >= 1 && kSubs * kSpan * kSpans == kFlattenTile,
                "spans must tile a plan tile");
  const int32_t tile = static_cast<int32_t>(blockIdx.x) / kSubs;
  const int32_t sub = static_cast<int32_t>(blockIdx.x) - tile * kSubs;
  const ParamDesc d = desc[tile_map[tile]];
  const int64_t start = static_cast<int64_t>(tile - d.tile_begin) * kFlattenTile +
                        static_cast<int64_t>(sub) * kSpan * kSpans;
  const int64_t left = d.numel - start;
  if (left <= 0) return;
  const int64_t cnt = left < int64_t(kSpan) * kSpans ? left : int64_t(kSpan) * kSpans;
  // blockDim.x / kBcastThreads groups copy the same span, each to its share
  // of the ranks: ring positions [g*p/G, (g+1)*p/G) in the rotated order.
  const int tid = static_cast<int>(threadIdx.x) % kBcastThreads;
  const int lane = static_cast<int>(threadIdx.x) & 63;
  static_assert(kBcastThreads % 64 == 0, "a group is whole waves");
  const int32_t groups = static_cast<int32_t>(blockDim.x) / kBcastThreads;
  // The group index is the same in every lane of a wave; saying so keeps
  // the store loop and its readlane rank indices in scalar registers (left
  // to the compiler, the loop ran under an exec mask with the lane index
  // re-read per store: 0.745 against 0.770 of peak on the GPT-2 sync).
  const int32_t g =
      __builtin_amdgcn_readfirstlane(static_cast<int32_t>(threadIdx.x) / kBcastThreads);
  const int32_t k0 = g * p / groups, k1 = (g + 1) * p / groups;
  const int32_t rot = store_rotation(p);
  // rank r's part, read from the device table (uniform: scalar loads)
  auto slice_mem = [&](int32_t r) {
    return static_cast<U *>(const_cast<void *>(ptrs[static_cast<int64_t>(r) * n_params +
                                                    d.param])) + start;
  };
  constexpr int64_t kPerSpan = int64_t(kBcastThreads) * kBcastVpt;  // vectors
  const int64_t nv = cnt * EB / kVecBytes;
  uint4 nxt[kBcastVpt];
  // Lane r of every wave loads rank r's address once; the vector path takes
  // it from that lane (readlane, in wave-uniform code only), so the p
  // addresses cost one vector load instead of p scalar loads.
  uintptr_t mine = 0;
  if (lane < p) {
    mine = reinterpret_cast<uintptr_t>(ptrs[static_cast<int64_t>(lane) * n_params + d.param]);
  }
  auto slice = [&](int32_t r) {
    const uint32_t lo = __builtin_amdgcn_readlane(static_cast<uint32_t>(mine), r);
    const uint32_t hi = __builtin_amdgcn_readlane(static_cast<uint32_t>(mine >> 32), r);
    return reinterpret_cast<U *>((static_cast<uint64_t>(hi) << 32) | lo) + start;
  };
  const bool aligned = __all(lane >= p || (mine + start * EB) % kVecBytes == 0);
  const U *src = slice(root);
  int64_t done = 0;
  if (aligned) {
    // (Loading the root's address separately with a scalar load, so that
    // this load could be issued before the p addresses arrive, was slower:
    // 0.68 against 0.77.)
#pragma unroll
    for (int u = 0; u < kBcastVpt; ++u) {
      const int64_t j = u * kBcastThreads + tid;
      nxt[u] = j < nv ? load_vec<kBcastNtLoad>(src, j) : make_uint4(0, 0, 0, 0);
    }
    for (int sp = 0; sp < kSpans; ++sp) {
      const int64_t j0 = sp * kPerSpan;
      if (j0 >= nv) break;
      uint4 x[kBcastVpt];
#pragma unroll
      for (int u = 0; u < kBcastVpt; ++u) x[u] = nxt[u];
      if (sp + 1 < kSpans) {
#pragma unroll
        for (int u = 0; u < kBcastVpt; ++u) {
          const int64_t j = j0 + kPerSpan + u * kBcastThreads + tid;
          nxt[u] = j < nv ? load_vec<kBcastNtLoad>(src, j) : make_uint4(0, 0, 0, 0);
        }
      }
      for (int32_t k = k0; k < k1; ++k) {
        const int32_t r = ring_rank(rot, k, p);
        if (r == root) continue;
        U *dst = slice(r);
#pragma unroll
        for (int u = 0; u < kBcastVpt; ++u) {
          const int64_t j = j0 + u * kBcastThreads + tid;
          if (j < nv) store_vec<kNtStore>(dst, j, x[u]);
        }
      }
    }
    done = nv * kVecBytes / EB;
  }
  for (int64_t i = done + tid; i < cnt; i += kBcastThreads) {
    const U v = global_ptr<U>(src)[i];
    for (int32_t k = k0; k < k1; ++k) {
      const int32_t r = ring_rank(rot, k, p);
      if (r != root) global_ptr<U>(slice_mem(r))[i] = v;
    }
  }
}

template <int EB>
ddp_status launch_bucket(const ParamDesc *desc, const int32_t *tile_map, int32_t tiles,
                         int64_t elems, int32_t n_params, const void *const *ptrs, int32_t p,
                         int32_t root, hipStream_t stream, CallTimer &timer, bool last) {
  const int64_t blocks = int64_t(tiles) * (kFlattenTile * EB / (kBcastThreads * kBcastVpt *
                                                                 kVecBytes * bcast_spans<EB>()));
  if (blocks > INT32_MAX) return fail(DDP_EINVAL, "ddp_broadcast_coalesced: bucket too large");
  const dim3 grid(static_cast<uint32_t>(blocks));
  // A launch holds at most 2^32 - 1 work-items along x.
  int32_t waves = fanout_waves(p - 1);
  while (waves > 1 && blocks * kBcastThreads * waves > int64_t(UINT32_MAX)) waves /= 2;
  if (blocks * kBcastThreads > int64_t(UINT32_MAX)) {
    return fail(DDP_EINVAL, "ddp_broadcast_coalesced: bucket too large");
  }
  const dim3 block(static_cast<uint32_t>(kBcastThreads * waves));
  const size_t lds = residency_lds(DDPSIM_BCAST_WGS_PER_CU);
  const char *what = "coalesced_broadcast_kernel launch";
  if (int64_t(p - 1) * elems * EB > DDPSIM_BCAST_NT_STORE_BYTES) {
    return launch_lds(coalesced_broadcast_kernel<EB, true>, grid, block, lds,
                      stream, timer, last, what, desc, tile_map, n_params, ptrs, p, root);
  }
  return launch_lds(coalesced_broadcast_kernel<EB, false>, grid, block, lds, stream,
                    timer, last, what, desc, tile_map, n_params, ptrs, p, root);
}

}  // namespace
}  // namespace ddpsim

using namespace ddpsim;

extern "C" ddp_status ddp_broadcast_coalesced(const ddp_plan *plan, int32_t p,
                                              void *const *d_tensor_ptrs, int32_t root,
                                              hipStream_t stream, ddp_comm_stats *stats) {
  clear_error();
  CallTimer timer = CallTimer::take();
  const char *what = "ddp_broadcast_coalesced";
  if (plan == nullptr) return fail(DDP_EINVAL, "%s: plan is NULL", what);
  ddp_status s = check_p(p, what);
  if (s != DDP_OK) return s;
  if (root < 0 || root >= p) return fail(DDP_ERANGE, "%s: root=%d outside [0, %d)", what, root, p);
  const int32_t nb = plan_num_buckets(plan);
  int32_t eb = 0, n_params = 0;
  int64_t total = 0;
  int32_t last = -1;
  bool uploaded = true;
  for (int32_t b = 0; b < nb; ++b) {
    int32_t first, count, tiles;
    int64_t elems;
    const void *table;
    const int32_t *tile_map;
    bool up;
    plan_bucket_info(plan, b, &first, &count, &tiles, &elems, &table, &tile_map, &n_params, &eb,
                     &up);
    uploaded = up;
    total += elems * eb;
    if (tiles > 0) last = b;
  }
  if (nb > 0 && !uploaded) return fail(DDP_ENOTREADY, "%s: call ddp_plan_upload first", what);
  if (last >= 0 && d_tensor_ptrs == nullptr) {
    return fail(DDP_EINVAL, "%s: tensor pointer table is NULL", what);
  }
  if (stats != nullptr) {
    int64_t rounds = 0;
    while ((int64_t(1) << rounds) < p) ++rounds;
    stats->steps = rounds * nb;
    stats->messages = int64_t(p - 1) * nb;
    stats->bytes_sent_per_rank = rounds * total;
    stats->bytes_recv_per_rank = p > 1 ? total : 0;
    stats->total_bytes = int64_t(p - 1) * total;
    stats->hbm_bytes = int64_t(p) * total;
  }
  if (p == 1 || last < 0) return DDP_OK;
  const void *const *ptrs = reinterpret_cast<const void *const *>(d_tensor_ptrs);
  for (int32_t b = 0; b <= last; ++b) {
    int32_t first, count, tiles;
    int64_t elems;
    const void *table;
    const int32_t *tile_map;
    bool up;
    plan_bucket_info(plan, b, &first, &count, &tiles, &elems, &table, &tile_map, &n_params, &eb,
                     &up);
    if (tiles == 0) continue;
    const ParamDesc *desc = static_cast<const ParamDesc *>(table) + first;
    const bool fin = b == last;
    switch (eb) {
      case 1: s = launch_bucket<1>(desc, tile_map, tiles, elems, n_params, ptrs, p, root, stream, timer, fin); break;
      case 2: s = launch_bucket<2>(desc, tile_map, tiles, elems, n_params, ptrs, p, root, stream, timer, fin); break;
      case 4: s = launch_bucket<4>(desc, tile_map, tiles, elems, n_params, ptrs, p, root, stream, timer, fin); break;
      default: s = launch_bucket<8>(desc, tile_map, tiles, elems, n_params, ptrs, p, root, stream, timer, fin); break;
    }
    if (s != DDP_OK) return s;
  }
  return DDP_OK;
}
