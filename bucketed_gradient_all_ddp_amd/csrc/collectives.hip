// collectives.hip -- standalone reduce-scatter, all-gather and broadcast over
// p simulated ranks in one GPU's HBM ("Collective Ops From Scratch", the
// list of primitives its implementation provides; "Data parallelism",
// section "The collective operations").
//
//   reduce-scatter  out[r] = average of chunk r summed over ranks, folded in
//                   the ring order of the pre-rotated schedule (rank r+1
//                   first). One pass: each input read once, each output
//                   written once.
//   all-gather      out[r] = in[0] || ... || in[p-1]: every shard is read
//                   once and written to all p outputs (its owner's slice is
//                   skipped when the call is in place).
//   broadcast       the source buffer is read once and written to the other
//                   p-1 ranks. The doubling tree's rounds exist only in the
//                   accounting: on one device every copy reads the same
//                   bytes, so the tree would only add passes.
#include <algorithm>
#include <cstring>

#include "fold.hpp"
#include "fold_waves.hpp"
#include "internal.hpp"

namespace ddpsim {
namespace {

// Reduce-scatter shapes. Up to DDPSIM_RS_NARROW_MAX_RANKS ranks: one-wave
// workgroups of one vector per lane, at most DDPSIM_RS_WGS_PER_CU of them
// resident per CU (8 ranks of 1 GiB: 5.59 -> 6.36 TB/s). More ranks: the
// wide shape below (at 64 ranks of 2 GiB the narrow one was 2% slower).
#ifndef DDPSIM_RS_THREADS
#define DDPSIM_RS_THREADS 256  // wide shape: threads per workgroup
#endif
#ifndef DDPSIM_RS_VPT
#define DDPSIM_RS_VPT 2  // wide shape: 16-byte vectors per thread
#endif
#ifndef DDPSIM_RS_NARROW_MAX_RANKS
#define DDPSIM_RS_NARROW_MAX_RANKS 16
#endif
#ifndef DDPSIM_RS_WGS_PER_CU
#define DDPSIM_RS_WGS_PER_CU 11
#endif
// Fan-out copy (all-gather, broadcast): tiles of one vector per lane across
// one wave (8 ranks of 1 GiB: all-gather 5.40 -> 5.83, broadcast 5.27 ->
// 5.77 TB/s against 256 threads x 4 vectors; at 64 ranks 1-4% better), each
// tile's destinations shared by the waves of its workgroup (fanout_waves). A
// bound on residency gained nothing here.
#ifndef DDPSIM_COPY_THREADS
#define DDPSIM_COPY_THREADS 64
#endif
#ifndef DDPSIM_COPY_VPT
#define DDPSIM_COPY_VPT 1
#endif
#ifndef DDPSIM_COPY_NT_BYTES
// Copies that write more than this in total use non-temporal stores (8
// ranks of 1 GiB: +2%; 64 ranks of 128 MiB: +5%); smaller outputs stay
// eligible for the Infinity Cache, where the next reader may find them.
#define DDPSIM_COPY_NT_BYTES (int64_t(256) << 20)
#endif
#ifndef DDPSIM_COPY_WGS_PER_CU
#define DDPSIM_COPY_WGS_PER_CU 0
#endif
#ifndef DDPSIM_RS_WAVE_RULE
#define DDPSIM_RS_WAVE_RULE 1  // 0: never split a tile's ranks over waves; 2, 8: W beyond 16 ranks
#endif
#ifndef DDPSIM_RS_WAVES_BYTES
#define DDPSIM_RS_WAVES_BYTES (int64_t(256) << 20)  // inputs past the Infinity Cache
#endif
#ifndef DDPSIM_RS_WAVES_SMALL_TILES
#define DDPSIM_RS_WAVES_SMALL_TILES 512  // calls of at most this many tiles are latency-bound
#endif
constexpr int kRsThreads = DDPSIM_RS_THREADS;
constexpr int kRsVpt = DDPSIM_RS_VPT;
constexpr int kRsNarrowThreads = 64;
constexpr int kRsRb = 8;
constexpr int kCopyThreads = DDPSIM_COPY_THREADS;  // fan-out copy workgroup
constexpr int kCopyVpt = DDPSIM_COPY_VPT;

// Reduce-scatter, C = n/p elements per shard. Workgroups of shard c:
// blockIdx.x / tiles_per_chunk. kVector: C is a whole number of 16-byte
// vectors, so input chunk c and output c are both vector aligned.
template <typename Tr, int VPT, int RB, bool kVector, int THR>
__global__ __launch_bounds__(THR) void reduce_scatter_kernel(
    RankTable in, RankTable out, int32_t p, int64_t C, int32_t tiles_per_chunk,
    Divide div) {
  constexpr int V = Tr::kVec;
  const int32_t c = static_cast<int32_t>(blockIdx.x) / tiles_per_chunk;
  const int32_t t = static_cast<int32_t>(blockIdx.x) - c * tiles_per_chunk;
  const int32_t first = c + 1 == p ? 0 : c + 1;
  void *dst = out.ptr[c];
  const int tid = static_cast<int>(threadIdx.x);
  if constexpr (kVector) {
    // tiles on the inputs' grid (p streams), the one output stream follows
    const int64_t nv = C / V;
    const int64_t v0 = static_cast<int64_t>(c) * nv, v1 = v0 + nv;
    const int64_t base = aligned_tile_base(v0, t, int64_t(THR) * VPT);
    if (base >= v1) return;
    int64_t vi[VPT];
    bool ok[VPT];
#pragma unroll
    for (int u = 0; u < VPT; ++u) {
      vi[u] = base + u * THR + tid;
      ok[u] = vi[u] >= v0 && vi[u] < v1;
    }
    float acc[VPT][V];
    fold_vectors<Tr, VPT, RB, true>(TablePtrs{in}, p, first, vi, ok, acc);
#pragma unroll
    for (int u = 0; u < VPT; ++u) {
      if (!ok[u]) continue;
#pragma unroll
      for (int e = 0; e < V; ++e) acc[u][e] = apply_divide(acc[u][e], div);
      store_vec<true>(dst, vi[u] - v0, Tr::narrow(acc[u]));
    }
  } else {
    // Element-wise path for shards that are not a whole number of vectors.
    const int64_t per_tile = int64_t(THR) * VPT * V;
    const int64_t lo = static_cast<int64_t>(t) * per_tile;
    for (int64_t j = lo + tid; j < lo + per_tile && j < C; j += THR) {
      const float y = apply_divide(fold_scalar<Tr>(TablePtrs{in}, p, first, c * C + j), div);
      Tr::store1(dst, j, y);
    }
  }
}

// The same reduce-scatter on the vector path with the ranks of a 64-vector
// tile split over the W waves of a workgroup (fold_tile_waves): one tile per
// workgroup, and the first wave stores the finished sum.
template <typename Tr, int W, int S>
__global__ __launch_bounds__(64 * W) void reduce_scatter_waves_kernel(
    RankTable in, RankTable out, int32_t p, int64_t C, int32_t tiles_per_chunk, Divide div) {
  extern __shared__ float lds[];
  constexpr int V = Tr::kVec;
  const int32_t c = static_cast<int32_t>(blockIdx.x) / tiles_per_chunk;
  const int32_t t = static_cast<int32_t>(blockIdx.x) - c * tiles_per_chunk;
  const int32_t first = c + 1 == p ? 0 : c + 1;
  const int lane = static_cast<int>(threadIdx.x) & 63;
  const int32_t wave = __builtin_amdgcn_readfirstlane(static_cast<int32_t>(threadIdx.x) >> 6);
  const int32_t lo = wave * p / W, hi = (wave + 1) * p / W;
  const int64_t nv = C / V;
  const int64_t v0 = static_cast<int64_t>(c) * nv, v1 = v0 + nv;
  const int64_t base = aligned_tile_base(v0, t, 64);
  if (base >= v1) return;  // workgroup-uniform
  const int64_t vi = base + lane;
  const bool ok = vi >= v0 && vi < v1;
  float acc[V];
  fold_tile_waves<Tr, W, S>(TablePtrs{in}, p, first, wave, lo, hi, vi, ok, lds, acc);
  if (wave != 0 || !ok) return;
#pragma unroll
  for (int e = 0; e < V; ++e) acc[e] = apply_divide(acc[e], div);
  store_vec<true>(out.ptr[c], vi - v0, Tr::narrow(acc));
}

// Copy `bytes` from each source s (blockIdx.y) to every destination r at
// byte offset s * dst_stride, except r == skip[s]. kVector: sources and
// destination offsets are 16-byte aligned; the last bytes % 16 are copied
// as 16-bit units (element sizes are 2 or 4 bytes).
struct SkipTable {
  int32_t rank[kMaxRanks];
};

// The workgroup is blockDim.x / kCopyThreads groups of kCopyThreads threads
// (one wave each at the default shape). Every group copies the same tile and
// stores it to its share of the destinations: ring positions [g*p/G,
// (g+1)*p/G) of the workgroup's rotated rank order (fanout_waves).
template <int VPT, bool kVector, bool kNtStore, bool kNtLoad>
__global__ __launch_bounds__(kCopyThreads * kMaxFanoutWaves) void fanout_copy_kernel(
    RankTable src, RankTable dst, int32_t p, int64_t bytes, int64_t dst_stride,
    SkipTable skip) {
  const int32_t s = static_cast<int32_t>(blockIdx.y);
  const int32_t no = skip.rank[s];
  const char *from = static_cast<const char *>(src.ptr[s]);
  const int64_t off = static_cast<int64_t>(s) * dst_stride;
  const int tid = static_cast<int>(threadIdx.x) % kCopyThreads;
  const int32_t groups = static_cast<int32_t>(blockDim.x) / kCopyThreads;
  // Left per-lane on purpose: each store then takes its destination address
  // with a vector load from the argument table, which the compiler issues
  // between stores. Declared wave-uniform, the loop instead waited on a
  // scalar load of the address before every store: 0.71 against 0.80 of
  // peak for 1 -> 7 at 1 GiB in a probe of both forms.
  const int32_t g = static_cast<int32_t>(threadIdx.x) / kCopyThreads;
  const int32_t k0 = g * p / groups, k1 = (g + 1) * p / groups;
  const int32_t rot = store_rotation(p);
  if constexpr (kVector) {
    // tiles on the destinations' grid (they are the many streams): source
    // s lands at s * dst_stride, so its tiles start `shift` vectors early
    const int64_t nv = bytes / 16;
    constexpr int64_t kTw = int64_t(kCopyThreads) * VPT;
    static_assert((kTw & (kTw - 1)) == 0, "tile width must be a power of two");
    const int64_t shift = (off / 16) & (kTw - 1);
    const int64_t base = static_cast<int64_t>(blockIdx.x) * kTw - shift;
    uint4 x[VPT];
    bool ok[VPT];
#pragma unroll
    for (int u = 0; u < VPT; ++u) {
      const int64_t j = base + u * kCopyThreads + tid;
      ok[u] = j >= 0 && j < nv;
      if (ok[u]) x[u] = load_vec<kNtLoad>(from, j);
    }
    for (int32_t k = k0; k < k1; ++k) {
      const int32_t r = ring_rank(rot, k, p);
      if (r == no) continue;
      char *to = static_cast<char *>(dst.ptr[r]) + off;
#pragma unroll
      for (int u = 0; u < VPT; ++u) {
        if (ok[u]) store_vec<kNtStore>(to, base + u * kCopyThreads + tid, x[u]);
      }
    }
    // trailing bytes, by the last workgroup
    if (blockIdx.x == gridDim.x - 1) {
      const int64_t tail = bytes - nv * 16;
      const int64_t units = tail / 2;
      if (tid < units) {
        const int64_t b = nv * 16 + 2 * tid;
        const uint16_t v = *reinterpret_cast<const uint16_t *>(from + b);
        for (int32_t k = k0; k < k1; ++k) {
          const int32_t r = ring_rank(rot, k, p);
          if (r == no) continue;
          *reinterpret_cast<uint16_t *>(static_cast<char *>(dst.ptr[r]) + off + b) = v;
        }
      }
    }
  } else {
    const int64_t units = bytes / 2;
    const int64_t per_tile = int64_t(kCopyThreads) * VPT * 8;
    const int64_t lo = static_cast<int64_t>(blockIdx.x) * per_tile;
    for (int64_t j = lo + tid; j < lo + per_tile && j < units; j += kCopyThreads) {
      const uint16_t v = reinterpret_cast<const uint16_t *>(from)[j];
      for (int32_t k = k0; k < k1; ++k) {
        const int32_t r = ring_rank(rot, k, p);
        if (r == no) continue;
        *reinterpret_cast<uint16_t *>(static_cast<char *>(dst.ptr[r]) + off + 2 * j) = v;
      }
    }
  }
}

// vec_ok: every source is 16-byte aligned (destinations always are).
ddp_status launch_fanout(const RankTable &src, int32_t n_src, bool vec_ok,
                         const RankTable &dst, int32_t p, int64_t bytes,
                         int64_t dst_stride, const SkipTable &skip,
                         hipStream_t stream, CallTimer &timer, const char *what) {
  if (bytes == 0) return DDP_OK;
  const bool vec = vec_ok && dst_stride % 16 == 0;
  // kCopyThreads * kCopyVpt vectors per workgroup in both paths
  const int64_t per_tile = int64_t(kCopyThreads) * kCopyVpt * 16;
  // one more tile when a source lands off the destinations' tile grid
  const int64_t tiles = std::max<int64_t>(
      1, ceil_div(bytes, per_tile) + (n_src > 1 && dst_stride % per_tile != 0 ? 1 : 0));
  const dim3 grid(static_cast<uint32_t>(tiles), static_cast<uint32_t>(n_src));
  const size_t lds = residency_lds(DDPSIM_COPY_WGS_PER_CU);
  const bool nt = int64_t(p) * n_src * bytes > DDPSIM_COPY_NT_BYTES;
  // Destinations per source vector: p, less one where a source's own rank
  // is skipped.
  int32_t dests = 0;
  for (int32_t s = 0; s < n_src; ++s) {
    dests = std::max(dests, p - (skip.rank[s] >= 0 ? 1 : 0));
  }
  // A launch holds at most 2^32 - 1 work-items along x.
  int32_t waves = fanout_waves(dests);
  while (waves > 1 && tiles * kCopyThreads * waves > int64_t(UINT32_MAX)) waves /= 2;
  if (tiles * kCopyThreads > int64_t(UINT32_MAX)) {
    return fail(DDP_EINVAL, "%s: buffer too large", what);
  }
  const dim3 block(static_cast<uint32_t>(kCopyThreads * waves));
  // A plain copy (every source byte written to one destination) also
  // streams its loads: 2 ranks of 1 GiB, 6.44 -> 6.66 TB/s. With more
  // destinations per read non-temporal loads lost 4% (8 ranks) and 6% (64),
  // and the waves of a workgroup would no longer find the source in cache.
  if (vec && nt && dests == 1) {
    return launch_lds(fanout_copy_kernel<kCopyVpt, true, true, true>, grid, block,
                      lds, stream, timer, true, what, src, dst, p, bytes, dst_stride, skip);
  }
  if (vec && nt) {
    return launch_lds(fanout_copy_kernel<kCopyVpt, true, true, false>, grid, block,
                      lds, stream, timer, true, what, src, dst, p, bytes, dst_stride, skip);
  }
  if (vec) {
    return launch_lds(fanout_copy_kernel<kCopyVpt, true, false, false>, grid, block,
                      lds, stream, timer, true, what, src, dst, p, bytes, dst_stride, skip);
  }
  return launch_lds(fanout_copy_kernel<kCopyVpt, false, false, false>, grid, block,
                    lds, stream, timer, true, what, src, dst, p, bytes, dst_stride, skip);
}

// Everything a reduce-scatter launch needs besides its shape.
struct RsLaunch {
  dim3 grid;
  hipStream_t stream;
  CallTimer *timer;
  RankTable in, out;
  int32_t p;
  int64_t C;
  int32_t tiles_per_chunk;
  Divide div;
};

template <int VPT, int THR, typename Tr, bool kVector>
ddp_status launch_rs_as(const RsLaunch &L, size_t lds) {
  return launch_lds(reduce_scatter_kernel<Tr, VPT, kRsRb, kVector, THR>, L.grid, dim3(THR), lds,
                    L.stream, *L.timer, true, "reduce_scatter_kernel launch", L.in, L.out, L.p,
                    L.C, L.tiles_per_chunk, L.div);
}

// Waves per tile of the reduce-scatter's split form for p ranks (1: the
// shapes above). Measured on identical buffers past the Infinity Cache
// against those shapes: 2 waves lost at 12 ranks (0.83 -> 0.75 of peak),
// were level at 16 and 17, and gained from 20 up (20-28 ranks 0.72-0.73 ->
// 0.80-0.82, 40 ranks 0.74 -> 0.79, 64 ranks 0.745 -> 0.79); 4 and 8 waves
// lost everywhere below 64 ranks and trailed 2 waves at 64.
// A small call (at most DDPSIM_RS_WAVES_SMALL_TILES tiles) is latency-bound
// and takes 8 waves from 17 ranks on: 64 ranks, shards of 64 and 1,024
// elements, 10.0 -> 4.6 and 15.6 -> 4.8 us per call (2 waves: 5.5, 5.8);
// 32 ranks 7.0 -> 4.1 us. Between the two regimes (inputs in the Infinity
// Cache, more tiles) the split gained nothing (2 waves) or lost (8 waves).
int32_t rs_waves(int32_t p, bool small) {
  if (!DDPSIM_RS_WAVE_RULE || p <= 16) return 1;
  if (small) return 8;
  if (DDPSIM_RS_WAVE_RULE == 2 || DDPSIM_RS_WAVE_RULE == 8) return DDPSIM_RS_WAVE_RULE;
  return 2;
}

template <int W>
ddp_status launch_rs_waves(const RsLaunch &L, int32_t dtype) {
  // the residency bound counts waves: ceil(bound / W) workgroups per CU
  const int32_t bound = fold_residency(DDPSIM_RS_WGS_PER_CU, L.p);
  const int vec = dtype == DDP_F32 ? F32Traits::kVec : BF16Traits::kVec;
  const size_t lds = std::max(residency_lds(bound > 0 ? (bound + W - 1) / W : 0),
                              size_t(64) * vec * sizeof(float));
  constexpr int kLarge = (kMaxRanks + W - 1) / W;
  constexpr int kSmall = kLarge < 8 ? kLarge : 8;
  const bool few = (L.p + W - 1) / W <= kSmall;
  const char *kname = "reduce_scatter_waves_kernel launch";
  const dim3 block(64 * W);
  if (dtype == DDP_F32) {
    if (few) {
      return launch_lds(reduce_scatter_waves_kernel<F32Traits, W, kSmall>, L.grid, block, lds,
                        L.stream, *L.timer, true, kname, L.in, L.out, L.p, L.C,
                        L.tiles_per_chunk, L.div);
    }
    return launch_lds(reduce_scatter_waves_kernel<F32Traits, W, kLarge>, L.grid, block, lds,
                      L.stream, *L.timer, true, kname, L.in, L.out, L.p, L.C, L.tiles_per_chunk,
                      L.div);
  }
  if (few) {
    return launch_lds(reduce_scatter_waves_kernel<BF16Traits, W, kSmall>, L.grid, block, lds,
                      L.stream, *L.timer, true, kname, L.in, L.out, L.p, L.C, L.tiles_per_chunk,
                      L.div);
  }
  return launch_lds(reduce_scatter_waves_kernel<BF16Traits, W, kLarge>, L.grid, block, lds,
                    L.stream, *L.timer, true, kname, L.in, L.out, L.p, L.C, L.tiles_per_chunk,
                    L.div);
}

template <int VPT, int THR>
ddp_status launch_rs(const RsLaunch &L, int32_t dtype, bool vec, size_t lds) {
  if (dtype == DDP_F32) {
    return vec ? launch_rs_as<VPT, THR, F32Traits, true>(L, lds)
               : launch_rs_as<VPT, THR, F32Traits, false>(L, lds);
  }
  return vec ? launch_rs_as<VPT, THR, BF16Traits, true>(L, lds)
             : launch_rs_as<VPT, THR, BF16Traits, false>(L, lds);
}

void fill_stats(ddp_comm_stats *st, int64_t steps, int64_t messages, int64_t sent,
                int64_t recv, int64_t total, int64_t hbm) {
  if (st == nullptr) return;
  st->steps = steps;
  st->messages = messages;
  st->bytes_sent_per_rank = sent;
  st->bytes_recv_per_rank = recv;
  st->total_bytes = total;
  st->hbm_bytes = hbm;
}

}  // namespace
}  // namespace ddpsim

using namespace ddpsim;

extern "C" ddp_status reduce_scatter_sim(const void *const *in, void *const *out,
                                         int32_t p, int64_t n, int32_t dtype,
                                         int32_t avg_mode, const int64_t *tokens,
                                         hipStream_t stream, ddp_comm_stats *stats) {
  clear_error();
  CallTimer timer = CallTimer::take();
  const char *what = "reduce_scatter_sim";
  ddp_status s = check_p(p, what);
  if (s != DDP_OK) return s;
  if (n < 0) return fail(DDP_EINVAL, "%s: n is negative", what);
  const int eb = elem_bytes_of(dtype);
  if (eb == 0) return fail(DDP_EINVAL, "%s: unknown dtype %d", what, dtype);
  if (n % p != 0) {
    return fail(DDP_ENOTDIVISIBLE, "%s: n=%lld is not divisible by p=%d", what,
                (long long)n, p);
  }
  Divide div;
  s = make_divide(avg_mode, p, tokens, &div);
  if (s != DDP_OK) return s;
  const int64_t C = n / p;
  s = check_rank_buffers(what, in, p, n * eb);
  if (s != DDP_OK) return s;
  s = check_rank_buffers(what, reinterpret_cast<const void *const *>(out), p, C * eb, eb);
  if (s != DDP_OK) return s;
  // out[r] may sit exactly on its own chunk of in[r]; nothing else may overlap.
  for (int32_t r = 0; r < p && C > 0; ++r) {
    const char *own = static_cast<const char *>(in[r]) + r * C * eb;
    for (int32_t q = 0; q < p; ++q) {
      if (!ranges_overlap(out[r], C * eb, in[q], n * eb)) continue;
      if (q == r && out[r] == own) continue;
      return fail(DDP_EALIAS, "%s: output of rank %d overlaps input of rank %d", what, r, q);
    }
  }
  fill_stats(stats, p - 1, int64_t(p) * (p - 1), (p - 1) * C * 4, (p - 1) * C * 4,
             int64_t(p) * (p - 1) * C * 4, (int64_t(p) + 1) * n * eb);
  if (n == 0) return DDP_OK;
  const RankTable tin = make_table(in, p);
  const RankTable tout = make_table(reinterpret_cast<const void *const *>(out), p);
  const int V = dtype == DDP_F32 ? 4 : 8;
  const bool vec = C % V == 0 && all_vec_aligned(reinterpret_cast<const void *const *>(out), p);
  const int64_t units = vec ? C / V : C;
  if (vec) {
    // tiles of 64 vectors on the inputs' grid, one more when chunks are off it
    const int64_t tpcw = std::max<int64_t>(1, ceil_div(units, 64) + (units % 64 != 0 ? 1 : 0));
    const int64_t bw = tpcw * p;
    const bool small = bw <= DDPSIM_RS_WAVES_SMALL_TILES;
    const int32_t waves = rs_waves(p, small);
    // past the Infinity Cache or latency-bound; a launch holds at most
    // 2^32 - 1 threads, and past that the shapes below run
    if (waves > 1 && (small || int64_t(p) * n * eb > DDPSIM_RS_WAVES_BYTES) &&
        bw * 64 * waves <= int64_t(UINT32_MAX)) {
      const RsLaunch Lw{dim3(static_cast<uint32_t>(bw)), stream, &timer, tin, tout, p, C,
                        static_cast<int32_t>(tpcw), div};
      return waves == 2 ? launch_rs_waves<2>(Lw, dtype) : launch_rs_waves<8>(Lw, dtype);
    }
  }
  const bool narrow = p <= DDPSIM_RS_NARROW_MAX_RANKS;
  const int64_t per_tile =
      (narrow ? int64_t(kRsNarrowThreads) : int64_t(kRsThreads) * kRsVpt) * (vec ? 1 : V);
  // one more tile when the chunks do not start on the vector path's tile grid
  const int64_t tpc =
      std::max<int64_t>(1, ceil_div(units, per_tile) + (vec && units % per_tile != 0 ? 1 : 0));
  const int64_t blocks = tpc * p;
  if (blocks > INT32_MAX) return fail(DDP_EINVAL, "%s: n too large", what);
  const RsLaunch L{dim3(static_cast<uint32_t>(blocks)), stream, &timer, tin, tout, p, C,
                   static_cast<int32_t>(tpc), div};
  if (narrow) {
    return launch_rs<1, kRsNarrowThreads>(L, dtype, vec, residency_lds(fold_residency(DDPSIM_RS_WGS_PER_CU, p)));
  }
  return launch_rs<kRsVpt, kRsThreads>(L, dtype, vec, 0);
}

extern "C" ddp_status allgather_sim(const void *const *in, void *const *out, int32_t p,
                                    int64_t n, int32_t dtype, hipStream_t stream,
                                    ddp_comm_stats *stats) {
  clear_error();
  CallTimer timer = CallTimer::take();
  const char *what = "allgather_sim";
  ddp_status s = check_p(p, what);
  if (s != DDP_OK) return s;
  if (n < 0) return fail(DDP_EINVAL, "%s: n is negative", what);
  const int eb = elem_bytes_of(dtype);
  if (eb == 0) return fail(DDP_EINVAL, "%s: unknown dtype %d", what, dtype);
  if (n % p != 0) {
    return fail(DDP_ENOTDIVISIBLE, "%s: n=%lld is not divisible by p=%d", what,
                (long long)n, p);
  }
  const int64_t C = n / p;
  s = check_rank_buffers(what, reinterpret_cast<const void *const *>(out), p, n * eb);
  if (s != DDP_OK) return s;
  if (in == nullptr) return fail(DDP_EINVAL, "%s: input array is NULL", what);
  SkipTable skip;
  for (int32_t r = 0; r < kMaxRanks; ++r) skip.rank[r] = -1;
  int64_t in_place = 0;
  for (int32_t j = 0; j < p && C > 0; ++j) {
    if (in[j] == nullptr) return fail(DDP_EINVAL, "%s: input of rank %d is NULL", what, j);
    if (reinterpret_cast<uintptr_t>(in[j]) % static_cast<uintptr_t>(eb) != 0) {
      return fail(DDP_EALIGN, "%s: input of rank %d is not %d-byte aligned", what, j, eb);
    }
    const char *slot = static_cast<const char *>(out[j]) + j * C * eb;
    if (in[j] == slot) {
      skip.rank[j] = j;
      ++in_place;
      for (int32_t r = 0; r < p; ++r) {
        if (r != j && ranges_overlap(in[j], C * eb, out[r], n * eb)) {
          return fail(DDP_EALIAS, "%s: input of rank %d overlaps output of rank %d", what, j, r);
        }
      }
      continue;
    }
    for (int32_t r = 0; r < p; ++r) {
      if (ranges_overlap(in[j], C * eb, out[r], n * eb)) {
        return fail(DDP_EALIAS, "%s: input of rank %d overlaps output of rank %d", what, j, r);
      }
    }
  }
  fill_stats(stats, p - 1, int64_t(p) * (p - 1), (p - 1) * C * eb, (p - 1) * C * eb,
             int64_t(p) * (p - 1) * C * eb, n * eb + (int64_t(p) * p - in_place) * C * eb);
  if (n == 0) return DDP_OK;
  return launch_fanout(make_table(in, p), p, all_vec_aligned(in, p),
                       make_table(reinterpret_cast<const void *const *>(out), p), p, C * eb,
                       C * eb, skip, stream, timer, "allgather fanout_copy_kernel launch");
}

extern "C" ddp_status broadcast_sim(void *const *bufs, int32_t p, int64_t n, int32_t src,
                                    int32_t dtype, hipStream_t stream,
                                    ddp_comm_stats *stats) {
  clear_error();
  CallTimer timer = CallTimer::take();
  const char *what = "broadcast_sim";
  ddp_status s = check_p(p, what);
  if (s != DDP_OK) return s;
  if (n < 0) return fail(DDP_EINVAL, "%s: n is negative", what);
  const int eb = elem_bytes_of(dtype);
  if (eb == 0) return fail(DDP_EINVAL, "%s: unknown dtype %d", what, dtype);
  if (src < 0 || src >= p) return fail(DDP_ERANGE, "%s: src=%d outside [0, %d)", what, src, p);
  s = check_rank_buffers(what, reinterpret_cast<const void *const *>(bufs), p, n * eb);
  if (s != DDP_OK) return s;
  int64_t rounds = 0;
  while ((int64_t(1) << rounds) < p) ++rounds;
  fill_stats(stats, rounds, p - 1, rounds * n * eb, p > 1 ? n * eb : 0,
             int64_t(p - 1) * n * eb, int64_t(p) * n * eb);
  if (n == 0 || p == 1) return DDP_OK;
  RankTable from;
  std::memset(&from, 0, sizeof from);
  from.ptr[0] = bufs[src];
  SkipTable skip;
  for (int32_t r = 0; r < kMaxRanks; ++r) skip.rank[r] = -1;
  skip.rank[0] = src;
  return launch_fanout(from, 1, true, make_table(reinterpret_cast<const void *const *>(bufs), p),
                       p, n * eb, 0, skip, stream, timer, "broadcast fanout_copy_kernel launch");
}
