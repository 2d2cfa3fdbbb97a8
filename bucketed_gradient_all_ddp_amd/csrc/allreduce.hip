// allreduce.hip -- ring all-reduce over p simulated ranks in one GPU's HBM.
//
// Two algorithms with identical results ("Collective Ops From Scratch",
// section "Ring allreduce in two passes"; "Data parallelism", section "Ring
// all-reduce, derived"):
//
//   FUSED  fused_allreduce_kernel: every workgroup owns a tile of one chunk c,
//          reads the tile from all p ranks once (16-byte loads, all of a batch
//          in flight), folds it in registers in the ring's order (rank c
//          first), averages, and writes the result to all p ranks. HBM traffic
//          2 p n bytes-per-element: the minimum for an in-place all-reduce.
//
//   RING   ring_step_kernel, launched 2(p-1) times: one launch is one ring
//          step in which every rank r "sends" one chunk to rank r+1, i.e. the
//          receiver's chunk is updated from the sender's copy in HBM
//          (reduce-scatter: add, all-gather: overwrite). Within a step no
//          rank reads a chunk another rank writes, so a step needs no
//          synchronisation beyond the launch boundary. The last
//          reduce-scatter step also averages each owner's finished chunk.
//          bf16 runs on an fp32 workspace (the partials are fp32).
//
// Padding to a multiple of p is virtual: chunks are [c C, (c+1) C) clipped
// to n, and elements past n are never read or written.
#include <algorithm>
#include <atomic>
#include <mutex>

#include "fold.hpp"
#include "fold_waves.hpp"
#include "internal.hpp"
#include "workspace.hpp"

namespace ddpsim {
namespace {

// ---------------------------------------------------------------------------
// Kernels
// ---------------------------------------------------------------------------

// Workgroup w handles tiles w, w + gridDim.x, ... (a grid-stride loop; the
// launches below give every tile a workgroup of its own); tile -> (chunk c,
// tile t within the chunk) = (tile / tiles_per_chunk, tile % tiles_per_chunk).
template <typename Tr, int VPT, int RB, bool kNT, int THR>
__global__ __launch_bounds__(THR) void fused_allreduce_kernel(
    RankTable bufs, int32_t p, int64_t n, int64_t C, int32_t tiles_per_chunk,
    Divide div) {
  constexpr int V = Tr::kVec;
  const int tid = static_cast<int>(threadIdx.x);
  const int64_t total = int64_t(tiles_per_chunk) * p;
  for (int64_t tile = blockIdx.x; tile < total; tile += gridDim.x) {
    const int32_t c = static_cast<int32_t>(tile / tiles_per_chunk);
    const int32_t t = static_cast<int32_t>(tile - int64_t(c) * tiles_per_chunk);
    const ChunkSpan k = chunk_span(c, C, n, V);
    if (k.s >= k.e) continue;

    // Up to V-1 unaligned elements on each side of the chunk: tile 0's
    // first lanes fold them one by one.
    if (t == 0 && tid >= THR - 2 * (V - 1)) {
      // the last wave's top lanes: for a short chunk the vector body sits in
      // the first wave, so the two run side by side
      const int lane = tid - (THR - 2 * (V - 1));
      const bool head = lane < V - 1;
      const int64_t i = head ? k.s + lane : k.tail_begin + (lane - (V - 1));
      if (i < (head ? k.head_end : k.e)) {
        const float y = apply_divide(fold_scalar<Tr>(TablePtrs{bufs}, p, c, i), div);
        for (int32_t r = 0; r < p; ++r) Tr::store1(bufs.ptr[r], i, y);
      }
    }

    const int64_t v0 = k.vs / V, v1 = k.ve / V;
    const int64_t base = aligned_tile_base(v0, t, int64_t(THR) * VPT);
    if (base >= v1) continue;
    int64_t vi[VPT];
    bool ok[VPT];
#pragma unroll
    for (int u = 0; u < VPT; ++u) {
      vi[u] = base + u * THR + tid;
      ok[u] = vi[u] >= v0 && vi[u] < v1;
    }
    float acc[VPT][V];
    fold_vectors<Tr, VPT, RB, kNT>(TablePtrs{bufs}, p, c, vi, ok, acc);
    uint4 y[VPT];
#pragma unroll
    for (int u = 0; u < VPT; ++u) {
#pragma unroll
      for (int e = 0; e < V; ++e) acc[u][e] = apply_divide(acc[u][e], div);
      y[u] = Tr::narrow(acc[u]);
    }
    const int32_t rot = store_rotation(p);
    for (int32_t k = 0; k < p; ++k) {
      void *dst = bufs.ptr[ring_rank(rot, k, p)];
#pragma unroll
      for (int u = 0; u < VPT; ++u) {
        if (ok[u]) store_vec<kNT>(dst, vi[u], y[u]);
      }
    }
  }
}

// The streaming form with the ranks of a tile split over the W waves of a
// workgroup (fold_tile_waves): workgroup = tile, wave w folds ring positions
// [w*p/W, (w+1)*p/W) of the tile (counted from rank c) after the waves
// before it, and stores the result to its share of the ranks.
template <typename Tr, int W, int S>
__global__ __launch_bounds__(64 * W) void fused_allreduce_waves_kernel(
    RankTable bufs, int32_t p, int64_t n, int64_t C, int32_t tiles_per_chunk, Divide div) {
  extern __shared__ float lds[];  // 64 * V floats (more when it bounds residency)
  constexpr int V = Tr::kVec;
  const int lane = static_cast<int>(threadIdx.x) & 63;
  const int32_t wave = __builtin_amdgcn_readfirstlane(static_cast<int32_t>(threadIdx.x) >> 6);
  const int32_t c = static_cast<int32_t>(blockIdx.x) / tiles_per_chunk;
  const int32_t t = static_cast<int32_t>(blockIdx.x) - c * tiles_per_chunk;
  const ChunkSpan k = chunk_span(c, C, n, V);
  if (k.s >= k.e) return;  // workgroup-uniform
  if (t == 0 && wave == 0 && lane >= 64 - 2 * (V - 1)) {
    const int e = lane - (64 - 2 * (V - 1));
    const bool head = e < V - 1;
    const int64_t i = head ? k.s + e : k.tail_begin + (e - (V - 1));
    if (i < (head ? k.head_end : k.e)) {
      const float y = apply_divide(fold_scalar<Tr>(TablePtrs{bufs}, p, c, i), div);
      for (int32_t r = 0; r < p; ++r) Tr::store1(bufs.ptr[r], i, y);
    }
  }
  const int64_t v0 = k.vs / V, v1 = k.ve / V;
  const int64_t base = aligned_tile_base(v0, t, 64);
  if (base >= v1) return;  // workgroup-uniform
  const int64_t vi = base + lane;
  const bool ok = vi >= v0 && vi < v1;
  const int32_t lo = wave * p / W, hi = (wave + 1) * p / W;
  float acc[V];
  fold_tile_waves<Tr, W, S>(TablePtrs{bufs}, p, c, wave, lo, hi, vi, ok, lds, acc);
#pragma unroll
  for (int e = 0; e < V; ++e) acc[e] = apply_divide(acc[e], div);
  const uint4 y = Tr::narrow(acc);
  if (!ok) return;
  const int32_t rot = store_rotation(p);
  for (int32_t r = lo; r < hi; ++r) store_vec<true>(bufs.ptr[ring_rank(rot, r, p)], vi, y);
}

// One ring step on p fp32 buffers. Sender r = blockIdx.x / tiles_per_chunk
// sends chunk (r + chunk_shift) mod p to rank r+1.
//   kReduce  receiver = receiver + sender (then divide, on the last
//            reduce-scatter step); otherwise receiver = sender.
// THR threads of VPT 16-byte vectors per workgroup; kNT makes the loads and
// stores non-temporal (buffers past the Infinity Cache).
template <bool kReduce, int VPT, int THR, bool kNT>
__global__ __launch_bounds__(THR) void ring_step_kernel(
    RankTable bufs, int32_t p, int32_t chunk_shift, int64_t n, int64_t C,
    int32_t tiles_per_chunk, Divide div) {
  constexpr int V = 4;
  const int32_t r = static_cast<int32_t>(blockIdx.x) / tiles_per_chunk;
  const int32_t t = static_cast<int32_t>(blockIdx.x) - r * tiles_per_chunk;
  const int32_t dst = r + 1 == p ? 0 : r + 1;
  const int32_t j = ring_rank(r, chunk_shift, p);
  const ChunkSpan k = chunk_span(j, C, n, V);
  if (k.s >= k.e) return;
  const float *src = static_cast<const float *>(bufs.ptr[r]);
  float *out = static_cast<float *>(bufs.ptr[dst]);
  const int tid = static_cast<int>(threadIdx.x);

  if (t == 0 && tid >= THR - 2 * (V - 1)) {
    const int lane = tid - (THR - 2 * (V - 1));
    const bool head = lane < V - 1;
    const int64_t i = head ? k.s + lane : k.tail_begin + (lane - (V - 1));
    if (i < (head ? k.head_end : k.e)) {
      out[i] = kReduce ? apply_divide(out[i] + src[i], div) : src[i];
    }
  }

  const int64_t v0 = k.vs / V, v1 = k.ve / V;
  const int64_t base = aligned_tile_base(v0, t, int64_t(THR) * VPT);
  if (base >= v1) return;
  uint4 a[VPT], b[VPT];
  int64_t vi[VPT];
  bool ok[VPT];
#pragma unroll
  for (int u = 0; u < VPT; ++u) {
    vi[u] = base + u * THR + tid;
    ok[u] = vi[u] >= v0 && vi[u] < v1;
    if (ok[u]) {
      b[u] = load_vec<kNT>(src, vi[u]);
      if (kReduce) a[u] = load_vec<kNT>(out, vi[u]);
    }
  }
#pragma unroll
  for (int u = 0; u < VPT; ++u) {
    if (!ok[u]) continue;
    if (kReduce) {
      float fa[4], fb[4];
      F32Traits::widen(a[u], fa);
      F32Traits::widen(b[u], fb);
#pragma unroll
      for (int e = 0; e < 4; ++e) fa[e] = apply_divide(fa[e] + fb[e], div);
      store_vec<kNT>(out, vi[u], F32Traits::narrow(fa));
    } else {
      store_vec<kNT>(out, vi[u], b[u]);
    }
  }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------

// Tuning of the fused kernel (compile-time; the defaults are the measured
// best on gfx950 for the gradient sets in the tests and benchmark).
#ifndef DDPSIM_FUSED_VPT
#define DDPSIM_FUSED_VPT 2  // 16-byte vectors per thread per tile
#endif
#ifndef DDPSIM_FUSED_THREADS
#define DDPSIM_FUSED_THREADS 256  // threads per workgroup
#endif
#ifndef DDPSIM_FUSED_RB
#define DDPSIM_FUSED_RB 8  // rank loads issued before their additions
#endif
#ifndef DDPSIM_FUSED_NT_BYTES
// Rank buffers larger than this in total use non-temporal loads and stores.
// Smaller ones may still sit in the 256 MB Infinity Cache (a bucket that
// ddp_flatten has just written, say), where ordinary accesses are faster.
#define DDPSIM_FUSED_NT_BYTES (int64_t(256) << 20)
#endif
#ifndef DDPSIM_FUSED_NT_WGS_PER_CU
// Buffers past the Infinity Cache take the in-place bucket kernel's shape:
// one-wave workgroups of one vector per lane, at most this many resident per
// CU (8 ranks of 1 GiB: 5.42 -> 6.06 TB/s against 256 threads x 2 vectors;
// 64 ranks of 2 GiB: equal). Cache-resident buffers keep the shape above.
#define DDPSIM_FUSED_NT_WGS_PER_CU 11
#endif
constexpr int kFusedVpt = DDPSIM_FUSED_VPT;
constexpr int kFusedRb = DDPSIM_FUSED_RB;
constexpr int kFusedThreads = DDPSIM_FUSED_THREADS;
constexpr int kFusedNtThreads = 64;
#ifndef DDPSIM_FUSED_SMALL_WAVES
// Small problems beyond 32 ranks take the 8-wave form: at 64 ranks a call on
// a tensor of 1,000 to 65,528 elements went from 12-14 us to 6-7 us (dispatch
// events included), the latency workload's 20,000 per-tensor calls replayed
// from a HIP graph from 336 to 270 ms.
#define DDPSIM_FUSED_SMALL_WAVES 1
#endif
#ifndef DDPSIM_FUSED_WAVE_RULE
#define DDPSIM_FUSED_WAVE_RULE 1  // 0: one wave per tile at every p; 2, 8: always W beyond 8 ranks
#endif
// Waves per tile of the streaming form for p ranks, measured on identical
// buffers against one wave: 1 up to 8 ranks (2 waves: -1% to +1.5% at 4-9
// ranks), 2 up to 27 (+4-7% at 12-24 ranks; 8 waves lost 3-18% there), 8
// from 28 (+6-11% at 28-64 ranks of 128-256 MiB, level at 64 of 2 GiB; 4
// waves trailed 2 or 8 at every count from 20 to 64).
int32_t fused_waves(int32_t p) {
  if (!DDPSIM_FUSED_WAVE_RULE || p <= 8) return 1;
  if (DDPSIM_FUSED_WAVE_RULE == 2 || DDPSIM_FUSED_WAVE_RULE == 8) return DDPSIM_FUSED_WAVE_RULE;
  return p < 28 ? 2 : 8;
}
// Small problems (few workgroups) are latency-bound: the fold's load batches
// run one after another, so there the kernel keeps 32 rank loads in flight
// per thread (one vector each) instead of 8.
constexpr int kSmallRb = 32;
constexpr int64_t kSmallBlocks = 512;
// Ring steps, each a copy or an add of one chunk per rank pair: one-wave
// workgroups of one 16-byte vector per lane in both shapes. At 8 ranks of
// 1 GiB, non-temporal accesses lifted a reduce-scatter step from 5.60 to
// 6.59 TB/s and an all-gather step from 5.76 to 6.56 (256 threads x 4
// vectors with ordinary accesses before; 256 x 1 and 64 x 2 both ~6.4); a
// residency bound cost 13-45% (16 and 11 workgroups per CU). On the GPT-2
// buckets (cache-resident) the one-wave shape with ordinary accesses gained
// 2% over 256 x 4; non-temporal accesses there lost 5%.
#ifndef DDPSIM_STEP_THREADS
#define DDPSIM_STEP_THREADS 64  // ring steps on cache-resident buffers
#endif
#ifndef DDPSIM_STEP_VPT
#define DDPSIM_STEP_VPT 1
#endif
constexpr int kStepVpt = DDPSIM_STEP_VPT;
constexpr int kStepThreads = DDPSIM_STEP_THREADS;
#ifndef DDPSIM_STEP_NT_BYTES
// Ring steps over rank buffers larger than this in total take the one-wave
// shape with non-temporal accesses (buffers past the Infinity Cache);
// smaller ones keep 256 threads x 4 vectors and ordinary accesses.
#define DDPSIM_STEP_NT_BYTES (int64_t(256) << 20)
#endif
#ifndef DDPSIM_STEP_NT_THREADS
#define DDPSIM_STEP_NT_THREADS 64
#endif
#ifndef DDPSIM_STEP_NT_VPT
#define DDPSIM_STEP_NT_VPT 1
#endif
#ifndef DDPSIM_STEP_NT_WGS_PER_CU
#define DDPSIM_STEP_NT_WGS_PER_CU 0  // workgroups resident per CU (0: no bound)
#endif
#ifndef DDPSIM_STEP_NT
#define DDPSIM_STEP_NT 1  // the large shape's accesses are non-temporal
#endif
constexpr int kStepNtThreads = DDPSIM_STEP_NT_THREADS;
constexpr int kStepNtVpt = DDPSIM_STEP_NT_VPT;
constexpr bool kStepNt = DDPSIM_STEP_NT != 0;


// Tiles per chunk of C elements: tiles of threads * vpt vectors on the grid
// of aligned_tile_base, one more when chunks do not start on that grid.
int32_t tiles_for(int64_t C, int vec, int vpt, int threads = kThreads) {
  const int64_t tw = int64_t(threads) * vpt;
  const int64_t vectors = C / vec;
  const bool aligned = C % (tw * vec) == 0;
  return static_cast<int32_t>(std::max<int64_t>(1, ceil_div(vectors, tw) + (aligned ? 0 : 1)));
}

template <int W>
ddp_status launch_fused_waves(const RankTable &tab, int32_t p, int64_t n, int64_t C, int32_t tpc,
                              int32_t dtype, const Divide &div, dim3 grid, hipStream_t stream,
                              CallTimer &timer) {
  const char *kname = "fused_allreduce_waves_kernel launch";
  // the residency bound counts waves: ceil(bound / W) workgroups per CU
  // (counted in workgroups it lost 3% at 8 ranks and 2% at 64)
  const int32_t bound = fold_residency(DDPSIM_FUSED_NT_WGS_PER_CU, p);
  const size_t lds_bound = residency_lds(bound > 0 ? (bound + W - 1) / W : 0);
  const int vec = dtype == DDP_F32 ? F32Traits::kVec : BF16Traits::kVec;
  const size_t lds = std::max(lds_bound, size_t(64) * vec * sizeof(float));
  constexpr int kLarge = W > 1 ? (kMaxRanks + W - 1) / W : 1;
  constexpr int kSmall = kLarge < 8 ? kLarge : 8;
  const bool few = (p + W - 1) / W <= kSmall;
  const dim3 block(64 * W);
  if (dtype == DDP_F32) {
    if (few) {
      return launch_lds(fused_allreduce_waves_kernel<F32Traits, W, kSmall>, grid, block, lds,
                        stream, timer, true, kname, tab, p, n, C, tpc, div);
    }
    return launch_lds(fused_allreduce_waves_kernel<F32Traits, W, kLarge>, grid, block, lds, stream,
                      timer, true, kname, tab, p, n, C, tpc, div);
  }
  if (few) {
    return launch_lds(fused_allreduce_waves_kernel<BF16Traits, W, kSmall>, grid, block, lds,
                      stream, timer, true, kname, tab, p, n, C, tpc, div);
  }
  return launch_lds(fused_allreduce_waves_kernel<BF16Traits, W, kLarge>, grid, block, lds, stream,
                    timer, true, kname, tab, p, n, C, tpc, div);
}

ddp_status launch_fused(const RankTable &tab, int32_t p, int64_t n, int32_t dtype,
                        const Divide &div, hipStream_t stream, CallTimer &timer) {
  const int64_t C = ceil_div(n, p);
  const int vec = dtype == DDP_F32 ? 4 : 8;
  const char *kname = "fused_allreduce_kernel launch";
  const bool nt = int64_t(p) * n * elem_bytes_of(dtype) > DDPSIM_FUSED_NT_BYTES;
  const int32_t tpc = tiles_for(C, vec, kFusedVpt, kFusedThreads);
  const int64_t blocks = int64_t(tpc) * p;
  if (blocks > INT32_MAX) return fail(DDP_EINVAL, "ring_allreduce_sim: n too large");
  if (DDPSIM_FUSED_SMALL_WAVES && p > kSmallRb && blocks * 2 <= kSmallBlocks) {
    // latency-bound with more ranks than one batch: every rank load of a
    // tile at once, split over 8 waves (64 ranks: one memory latency, not two)
    const int32_t tpcn = tiles_for(C, vec, 1, kFusedNtThreads);
    const dim3 gridn(static_cast<uint32_t>(int64_t(tpcn) * p));
    const size_t lds = size_t(64) * vec * sizeof(float);
    if (dtype == DDP_F32) {
      return launch_lds(fused_allreduce_waves_kernel<F32Traits, 8, 8>, gridn, dim3(512), lds,
                        stream, timer, true, kname, tab, p, n, C, tpcn, div);
    }
    return launch_lds(fused_allreduce_waves_kernel<BF16Traits, 8, 8>, gridn, dim3(512), lds,
                      stream, timer, true, kname, tab, p, n, C, tpcn, div);
  }
  if (p > kFusedRb && blocks * 2 <= kSmallBlocks) {
    // latency-bound: one vector per thread, 32 loads in flight
    const int32_t tpc1 = tiles_for(C, vec, 1);
    const dim3 grid1(static_cast<uint32_t>(int64_t(tpc1) * p));
    if (dtype == DDP_F32) {
      return launch(fused_allreduce_kernel<F32Traits, 1, kSmallRb, false, kThreads>, grid1,
                    dim3(kThreads), stream, timer, true, kname, tab, p, n, C, tpc1, div);
    }
    return launch(fused_allreduce_kernel<BF16Traits, 1, kSmallRb, false, kThreads>, grid1,
                  dim3(kThreads), stream, timer, true, kname, tab, p, n, C, tpc1, div);
  }
  const int32_t waves = fused_waves(p);
  if (nt && waves > 1) {
    const int32_t tpcn = tiles_for(C, vec, 1, kFusedNtThreads);
    const int64_t bn = int64_t(tpcn) * p;
    // a launch holds at most 2^32 - 1 threads; past that the one-wave form runs
    if (bn * kFusedNtThreads * waves <= int64_t(UINT32_MAX)) {
      const dim3 gridn(static_cast<uint32_t>(bn));
      return waves == 2
                 ? launch_fused_waves<2>(tab, p, n, C, tpcn, dtype, div, gridn, stream, timer)
                 : launch_fused_waves<8>(tab, p, n, C, tpcn, dtype, div, gridn, stream, timer);
    }
  }
  if (nt) {
    const int32_t tpcn = tiles_for(C, vec, 1, kFusedNtThreads);
    const int64_t bn = int64_t(tpcn) * p;
    if (bn > INT32_MAX) return fail(DDP_EINVAL, "ring_allreduce_sim: n too large");
    const dim3 gridn(static_cast<uint32_t>(bn));
    const size_t lds = residency_lds(fold_residency(DDPSIM_FUSED_NT_WGS_PER_CU, p));
    if (dtype == DDP_F32) {
      return launch_lds(fused_allreduce_kernel<F32Traits, 1, kFusedRb, true, kFusedNtThreads>,
                        gridn, dim3(kFusedNtThreads), lds, stream, timer, true, kname, tab, p, n,
                        C, tpcn, div);
    }
    return launch_lds(fused_allreduce_kernel<BF16Traits, 1, kFusedRb, true, kFusedNtThreads>,
                      gridn, dim3(kFusedNtThreads), lds, stream, timer, true, kname, tab, p, n, C,
                      tpcn, div);
  }
  const dim3 grid(static_cast<uint32_t>(blocks));
  const dim3 block(kFusedThreads);
  if (dtype == DDP_F32) {
    return launch(fused_allreduce_kernel<F32Traits, kFusedVpt, kFusedRb, false, kFusedThreads>,
                  grid, block, stream, timer, true, kname, tab, p, n, C, tpc, div);
  }
  return launch(fused_allreduce_kernel<BF16Traits, kFusedVpt, kFusedRb, false, kFusedThreads>,
                grid, block, stream, timer, true, kname, tab, p, n, C, tpc, div);
}

// Launch ring steps [first, first + count) on fp32 buffers, in one of two
// shapes (the same arithmetic).
template <int VPT, int THR, bool kNT>
ddp_status launch_steps_as(const RankTable &tab, int32_t p, int64_t n, const Divide &div,
                           int32_t first, int32_t count, hipStream_t stream, CallTimer &timer,
                           bool ends_call, size_t lds) {
  const int64_t C = ceil_div(n, p);
  const int32_t tpc = tiles_for(C, 4, VPT, THR);
  const int64_t blocks = int64_t(tpc) * p;
  if (blocks > INT32_MAX) return fail(DDP_EINVAL, "ring step: n too large");
  const Divide none{kNone, 1.0f, 1.0f};
  const dim3 grid(static_cast<uint32_t>(blocks));
  for (int32_t s = first; s < first + count; ++s) {
    const bool last = ends_call && s == first + count - 1;
    ddp_status st;
    if (s < p - 1) {
      const int32_t k = s;  // reduce-scatter step k: rank r sends chunk r - k
      const int32_t shift = ((-k) % p + p) % p;
      const Divide &d = (k == p - 2) ? div : none;
      st = launch_lds(ring_step_kernel<true, VPT, THR, kNT>, grid, dim3(THR), lds, stream, timer,
                      last, "ring_step_kernel launch", tab, p, shift, n, C, tpc, d);
    } else {
      const int32_t k = s - (p - 1);  // all-gather step k: chunk r + 1 - k
      const int32_t shift = ((1 - k) % p + p) % p;
      st = launch_lds(ring_step_kernel<false, VPT, THR, kNT>, grid, dim3(THR), lds, stream,
                      timer, last, "ring_step_kernel launch", tab, p, shift, n, C, tpc, none);
    }
    if (st != DDP_OK) return st;
  }
  return DDP_OK;
}

ddp_status launch_steps(const RankTable &tab, int32_t p, int64_t n, const Divide &div,
                        int32_t first, int32_t count, hipStream_t stream, CallTimer &timer,
                        bool ends_call) {
  if (int64_t(p) * n * 4 > DDPSIM_STEP_NT_BYTES) {
    return launch_steps_as<kStepNtVpt, kStepNtThreads, kStepNt>(
        tab, p, n, div, first, count, stream, timer, ends_call,
        residency_lds(DDPSIM_STEP_NT_WGS_PER_CU));
  }
  return launch_steps_as<kStepVpt, kStepThreads, false>(tab, p, n, div, first, count, stream,
                                                        timer, ends_call, 0);
}


void fill_allreduce_stats(ddp_comm_stats *st, int32_t p, int64_t n, int32_t dtype,
                          int32_t algo) {
  if (st == nullptr) return;
  const int64_t eb = elem_bytes_of(dtype);
  const int64_t C = n > 0 ? ceil_div(n, p) : 0;
  st->steps = 2 * int64_t(p - 1);
  st->messages = 2 * int64_t(p) * (p - 1);
  st->bytes_sent_per_rank = 2 * int64_t(p - 1) * C * 4;
  st->bytes_recv_per_rank = st->bytes_sent_per_rank;
  st->total_bytes = st->messages * C * 4;
  if (algo == DDP_ALGO_FUSED || p == 1) {
    st->hbm_bytes = 2 * int64_t(p) * n * eb;
  } else {
    int64_t b = 5 * int64_t(p - 1) * n * 4;
    if (dtype == DDP_BF16) b += 2 * int64_t(p) * n * (2 + 4);
    st->hbm_bytes = b;
  }
}


}  // namespace
}  // namespace ddpsim

using namespace ddpsim;

extern "C" size_t ring_allreduce_sim_workspace(int32_t p, int64_t n, int32_t dtype,
                                               int32_t algo) {
  if (p < 1 || p > kMaxRanks || n <= 0) return 0;
  if (algo != DDP_ALGO_RING || dtype != DDP_BF16 || p == 1) return 0;
  return static_cast<size_t>(p) * workspace_stride_elems(n) * 4;
}

namespace ddpsim {
namespace {

// The whole of ring_allreduce_sim after its timing request was taken: the
// workspace is the caller's, or the device's scratch array below.
ddp_status run_allreduce(void *const *bufs, int32_t p, int64_t n, int32_t dtype,
                         int32_t avg_mode, const int64_t *tokens, int32_t algo,
                         void *workspace, size_t workspace_bytes, hipStream_t stream,
                         ddp_comm_stats *stats, CallTimer &timer, const char *what) {
  Divide div;
  ddp_status s = validate_allreduce(bufs, p, n, dtype, avg_mode, tokens, &div, what);
  if (s != DDP_OK) return s;
  if (algo != DDP_ALGO_FUSED && algo != DDP_ALGO_RING) {
    return fail(DDP_EINVAL, "%s: unknown algorithm %d", what, algo);
  }
  const size_t need = ring_allreduce_sim_workspace(p, n, dtype, algo);
  s = check_workspace(what, workspace, workspace_bytes, need, bufs, p, n * elem_bytes_of(dtype));
  if (s != DDP_OK) return s;
  fill_allreduce_stats(stats, p, n, dtype, algo);
  if (n == 0) return DDP_OK;
  const RankTable tab = make_table(bufs, p);
  if (algo == DDP_ALGO_FUSED || p == 1) return launch_fused(tab, p, n, dtype, div, stream, timer);
  if (dtype == DDP_F32) return launch_steps(tab, p, n, div, 0, 2 * (p - 1), stream, timer, true);

  // bf16 ring: widen into fp32 rows, run the steps there, round back.
  const int64_t stride = workspace_stride_elems(n);
  float *ws = static_cast<float *>(workspace);
  const int32_t tpr = static_cast<int32_t>(ceil_div(ceil_div(n, 8), kThreads));
  const int64_t blocks = int64_t(tpr) * p;
  if (blocks > INT32_MAX) return fail(DDP_EINVAL, "%s: n too large", what);
  const dim3 grid(static_cast<uint32_t>(blocks));
  s = launch(bf16_workspace_kernel<true>, grid, dim3(kThreads), stream, timer, false,
             "bf16_workspace_kernel launch", tab, ws, stride, n, tpr);
  if (s != DDP_OK) return s;
  RankTable rows;
  for (int32_t r = 0; r < kMaxRanks; ++r) rows.ptr[r] = r < p ? ws + r * stride : nullptr;
  s = launch_steps(rows, p, n, div, 0, 2 * (p - 1), stream, timer, false);
  if (s != DDP_OK) return s;
  return launch(bf16_workspace_kernel<false>, grid, dim3(kThreads), stream, timer, true,
                "bf16_workspace_kernel launch", tab, ws, stride, n, tpr);
}

// Device memory that ring_allreduce_sim_noalloc uses as its workspace: the
// fp32 rows of a bf16 ring. Each GPU holds its own copy from the moment the
// library's code is loaded on it until the process ends. On the host the
// name is only a stand-in for the symbol; its device address comes from
// hipGetSymbolAddress, once per device (scratch_on_current_device).
static __device__ __align__(256) unsigned char scratch[DDP_NOALLOC_SCRATCH_BYTES];

constexpr int kScratchDevices = 64;
std::atomic<void *> g_scratch_of[kScratchDevices];
std::mutex g_scratch_mu;

// The current device's copy of `scratch` (its device address, looked up
// once per device and kept).
ddp_status scratch_on_current_device(const char *what, void **out) {
  int dev = -1;
  ddp_status s = check_hip(hipGetDevice(&dev), "hipGetDevice");
  if (s != DDP_OK) return s;
  if (dev < 0 || dev >= kScratchDevices) {
    return fail(DDP_ERANGE, "%s: device %d beyond the %d this library keeps scratch for", what,
                dev, kScratchDevices);
  }
  void *ptr = g_scratch_of[dev].load(std::memory_order_acquire);
  if (ptr == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    ptr = g_scratch_of[dev].load(std::memory_order_relaxed);
    if (ptr == nullptr) {
      s = check_hip(hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)), "hipGetSymbolAddress");
      if (s != DDP_OK) return s;
      if (ptr == nullptr) {
        return fail(DDP_EHIP, "%s: hipGetSymbolAddress gave no address for the scratch array",
                    what);
      }
      g_scratch_of[dev].store(ptr, std::memory_order_release);
    }
  }
  *out = ptr;
  return DDP_OK;
}

}  // namespace
}  // namespace ddpsim

extern "C" ddp_status ring_allreduce_sim(void *const *bufs, int32_t p, int64_t n,
                                         int32_t dtype, int32_t avg_mode,
                                         const int64_t *tokens, int32_t algo,
                                         void *workspace, size_t workspace_bytes,
                                         hipStream_t stream, ddp_comm_stats *stats) {
  clear_error();
  CallTimer timer = CallTimer::take();
  return run_allreduce(bufs, p, n, dtype, avg_mode, tokens, algo, workspace, workspace_bytes,
                       stream, stats, timer, "ring_allreduce_sim");
}

extern "C" ddp_status ring_allreduce_sim_noalloc(void *const *bufs, int32_t p, int64_t n,
                                                 int32_t dtype, int32_t avg_mode,
                                                 const int64_t *tokens, int32_t algo,
                                                 hipStream_t stream, ddp_comm_stats *stats) {
  clear_error();
  CallTimer timer = CallTimer::take();
  const char *what = "ring_allreduce_sim_noalloc";
  const size_t need = ring_allreduce_sim_workspace(p, n, dtype, algo);
  if (need > size_t(DDP_NOALLOC_SCRATCH_BYTES)) {
    return fail(DDP_EWORKSPACE,
                "%s: needs %zu bytes of workspace, more than the %lld of the device's scratch "
                "array (p=%d, n=%lld); use ring_allreduce_sim with a workspace",
                what, need, (long long)DDP_NOALLOC_SCRATCH_BYTES, p, (long long)n);
  }
  void *ws = nullptr;
  if (need > 0) {
    const ddp_status s = scratch_on_current_device(what, &ws);
    if (s != DDP_OK) return s;
  }
  return run_allreduce(bufs, p, n, dtype, avg_mode, tokens, algo, ws,
                       need > 0 ? size_t(DDP_NOALLOC_SCRATCH_BYTES) : 0, stream, stats, timer,
                       what);
}

extern "C" ddp_status ring_allreduce_sim_steps(void *const *bufs, int32_t p, int64_t n,
                                               int32_t avg_mode, const int64_t *tokens,
                                               int32_t first_step, int32_t n_steps,
                                               hipStream_t stream) {
  clear_error();
  CallTimer timer = CallTimer::take();
  Divide div;
  ddp_status s = validate_allreduce(bufs, p, n, DDP_F32, avg_mode, tokens, &div,
                                 "ring_allreduce_sim_steps");
  if (s != DDP_OK) return s;
  if (p < 2) return fail(DDP_ERANGE, "ring_allreduce_sim_steps: needs p >= 2");
  const int32_t total = 2 * (p - 1);
  if (first_step < 0 || n_steps < 0 || first_step > total || n_steps > total - first_step) {
    return fail(DDP_ERANGE, "ring_allreduce_sim_steps: steps [%d, %d) outside [0, %d)",
                first_step, first_step + n_steps, total);
  }
  if (n == 0 || n_steps == 0) return DDP_OK;
  return launch_steps(make_table(bufs, p), p, n, div, first_step, n_steps, stream, timer, true);
}
