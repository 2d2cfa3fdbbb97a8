// schedules.hip -- all-reduce under the logarithmic-latency schedules ("Data
// parallelism", section "Latency, trees, and choosing an algorithm"; the
// tree all-reduce of "Collective Ops From Scratch"), over p simulated ranks
// in one GPU's HBM, and the choice of a schedule by message size.
//
// Every one of these schedules sums each element as a pairwise tree over the
// ranks: both partners of an exchange compute a + b, the same number, so the
// pairing alone fixes the bits, and it is the same for every element. With
// q the largest power of two <= p, leaf v < q is x[v] (+ x[v+q] when that
// rank exists); recursive doubling then pairs leaves at distance 1, 2, 4, ...
// and Rabenseifner's halving and the tree's reduction pair them at distance
// q/2, q/4, ..., 1.
//
//   fused   tree_allreduce_kernel: each thread reads one 16-byte vector of
//           every rank, eight ranks at a time, sums the leaves in the
//           schedule's pairing (complete subtrees per batch of eight, joined
//           like a binary counter; leaves in natural or bit-reversed order),
//           divides, and writes all p ranks. 2 p n bytes-per-element of HBM
//           traffic.
//   steps   schedule_step_kernel, one launch per step of the literal
//           schedule: a step is a list of jobs (destination rank, source
//           rank, element range) that add, copy, or add pairwise into both
//           ranks. Jobs of one step never write what another job of the
//           step reads, so the launch boundary is the only synchronisation.
#include <algorithm>
#include <cmath>
#include <vector>

#include "internal.hpp"
#include "workspace.hpp"

namespace ddpsim {
namespace {

constexpr int ilog2(int q) { return q <= 1 ? 0 : 1 + ilog2(q / 2); }

// Reverse the low k bits of t.
constexpr int bit_reverse(int t, int k) {
  int r = 0;
  for (int i = 0; i < k; ++i) r |= ((t >> i) & 1) << (k - 1 - i);
  return r;
}

// ---------------------------------------------------------------------------
// Fused form
// ---------------------------------------------------------------------------

// The complete subtree of visit-order batch m (leaves m*RB .. m*RB+RB-1 in
// visit order, each with its extra rank folded in first).
template <int Q, bool kHalvingFirst, int W, typename LeafLoad>
__device__ __forceinline__ void tree_batch(const LeafLoad &leaf, int32_t extra, int m,
                                           float (&s)[W]) {
  constexpr int K = ilog2(Q);
  constexpr int RB = Q < 8 ? Q : 8;
  constexpr int KB = ilog2(RB);
  constexpr int B = Q / RB;
  // p < 2Q, so with Q at the rank limit there are no extra ranks
  constexpr bool kExtras = Q < kMaxRanks;
  int low = 0;  // the visit-order batch number's contribution to the leaf index
  if constexpr (B > 1) {
    low = kHalvingFirst ? static_cast<int>(__builtin_bitreverse32(static_cast<uint32_t>(m)) >>
                                           (32 - (K - KB)))
                        : m * RB;
  }
  float x[RB][W], y[RB][W];
#pragma unroll
  for (int j = 0; j < RB; ++j) {
    const int u = kHalvingFirst ? (bit_reverse(j, KB) << (K - KB)) + low : low + j;
    leaf(u, x[j]);
    if (kExtras && u < extra) leaf(u + Q, y[j]);
  }
#pragma unroll
  for (int j = 0; j < RB; ++j) {
    const int u = kHalvingFirst ? (bit_reverse(j, KB) << (K - KB)) + low : low + j;
    if (kExtras && u < extra) {
#pragma unroll
      for (int e = 0; e < W; ++e) x[j][e] = x[j][e] + y[j][e];
    }
  }
#pragma unroll
  for (int d = 1; d < RB; d *= 2) {
#pragma unroll
    for (int j = 0; j < RB; j += 2 * d) {
#pragma unroll
      for (int e = 0; e < W; ++e) x[j][e] = x[j][e] + x[j + d][e];
    }
  }
#pragma unroll
  for (int e = 0; e < W; ++e) s[e] = x[0][e];
}

// Leaves are visited in order t = 0..Q-1: leaf index t (recursive doubling,
// nearest neighbours first) or the bit reversal of t over log2 Q bits (q/2
// apart first). The balanced pairwise tree over that visit order is built
// in batches of RB = min(Q, 8) consecutive visits: the batch's RB loads are
// all issued before its additions, its leaves are summed as a complete
// subtree, and the batch sum joins the earlier batches like a binary
// counter (pending sums of 1, 2 and 4 batches in c[0..2]). The batch loop is
// not unrolled, so a thread holds one batch of vectors at a time.
template <int Q, bool kHalvingFirst, int W, typename LeafLoad>
__device__ __forceinline__ void tree_fold(const LeafLoad &leaf, int32_t extra,
                                          float (&out)[W]) {
  constexpr int RB = Q < 8 ? Q : 8;
  constexpr int B = Q / RB;
  float c[3][W];
#pragma unroll 1
  for (int m = 0; m < B; ++m) {
    float s[W];
    tree_batch<Q, kHalvingFirst>(leaf, extra, m, s);
    if (m & 1) {
#pragma unroll
      for (int e = 0; e < W; ++e) s[e] = c[0][e] + s[e];
      if (m & 2) {
#pragma unroll
        for (int e = 0; e < W; ++e) s[e] = c[1][e] + s[e];
        if (m & 4) {
#pragma unroll
          for (int e = 0; e < W; ++e) s[e] = c[2][e] + s[e];
        } else {
#pragma unroll
          for (int e = 0; e < W; ++e) c[2][e] = s[e];
        }
      } else {
#pragma unroll
        for (int e = 0; e < W; ++e) c[1][e] = s[e];
      }
    } else {
#pragma unroll
      for (int e = 0; e < W; ++e) c[0][e] = s[e];
    }
    if (m == B - 1) {
#pragma unroll
      for (int e = 0; e < W; ++e) out[e] = s[e];
    }
  }
}

// Leaf loaders: one 16-byte vector of rank u, widened; or one element.
template <typename Tr, bool kNT>
struct VectorLeaf {
  const RankTable &bufs;
  int64_t v;
  __device__ __forceinline__ void operator()(int u, float (&w)[Tr::kVec]) const {
    Tr::widen(load_vec<kNT>(bufs.ptr[u], v), w);
  }
};
template <typename Tr>
struct ElementLeaf {
  const RankTable &bufs;
  int64_t i;
  __device__ __forceinline__ void operator()(int u, float (&w)[1]) const {
    w[0] = Tr::load1(bufs.ptr[u], i);
  }
};

// A vector leaf for lanes that may lie past the last vector (those load
// nothing and fold zeros that are never stored).
template <typename Tr, bool kNT>
struct MaskedVectorLeaf {
  const RankTable &bufs;
  int64_t v;
  bool ok;
  __device__ __forceinline__ void operator()(int u, float (&w)[Tr::kVec]) const {
    Tr::widen(ok ? load_vec<kNT>(bufs.ptr[u], v) : make_uint4(0, 0, 0, 0), w);
  }
};

// One thread per 16-byte vector; thread nv (one past the last vector) folds
// the fewer-than-V tail elements one by one. Ranks Q..p-1 (extra = p - Q of
// them) are folded into ranks 0..extra-1 first.
// One-wave workgroups, at most DDPSIM_TREE_WGS_PER_CU resident per CU
// (Rabenseifner order, 8 ranks of 1 GiB: 5.61 -> 5.99 TB/s, 64 ranks of
// 128 MiB: 4.71 -> 5.20, 64 ranks of 2 GiB: equal, against 256 threads and
// full residency).
#ifndef DDPSIM_TREE_THREADS
#define DDPSIM_TREE_THREADS 64
#endif
#ifndef DDPSIM_TREE_WGS_PER_CU
#define DDPSIM_TREE_WGS_PER_CU 11
#endif
constexpr int kTreeThreads = DDPSIM_TREE_THREADS;

template <typename Tr, int Q, bool kHalvingFirst, bool kNT>
__global__ __launch_bounds__(kTreeThreads) void tree_allreduce_kernel(RankTable bufs, int32_t p,
                                                                  int64_t n, Divide div) {
  constexpr int V = Tr::kVec;
  const int32_t extra = p - Q;
  const int64_t nv = n / V;
  const int64_t g = static_cast<int64_t>(blockIdx.x) * kTreeThreads + threadIdx.x;
  if (g < nv) {
    float acc[V];
    tree_fold<Q, kHalvingFirst>(VectorLeaf<Tr, kNT>{bufs, g}, extra, acc);
#pragma unroll
    for (int e = 0; e < V; ++e) acc[e] = apply_divide(acc[e], div);
    const uint4 y = Tr::narrow(acc);
    const int32_t rot = store_rotation(p);
    for (int32_t k = 0; k < p; ++k) store_vec<kNT>(bufs.ptr[ring_rank(rot, k, p)], g, y);
  } else if (g == nv) {
    for (int64_t i = nv * V; i < n; ++i) {
      float acc[1];
      tree_fold<Q, kHalvingFirst>(ElementLeaf<Tr>{bufs, i}, extra, acc);
      const float y = apply_divide(acc[0], div);
      for (int32_t r = 0; r < p; ++r) Tr::store1(bufs.ptr[r], i, y);
    }
  }
}

// The streaming form for Q >= 16 with the batches of a tile split over the
// Q / 8 waves of a workgroup: wave m sums batch m (a complete subtree of 8
// visit-order leaves), the batch sums meet in LDS, and every wave joins them
// the way the binary counter above does (earlier + later at every level of
// a balanced tree over the batches), then stores the result to its share of
// the ranks. Same bits as tree_allreduce_kernel. lds holds Q / 8 * 64 * V
// floats.
template <typename Tr, int Q, bool kHalvingFirst>
__global__ __launch_bounds__(8 * Q) void tree_allreduce_waves_kernel(RankTable bufs, int32_t p,
                                                                    int64_t n, Divide div) {
  extern __shared__ float lds[];
  constexpr int V = Tr::kVec;
  constexpr int W = Q / 8;
  static_assert(Q >= 16 && W * 8 == Q, "one batch of 8 leaves per wave");
  const int lane = static_cast<int>(threadIdx.x) & 63;
  const int32_t wave = __builtin_amdgcn_readfirstlane(static_cast<int32_t>(threadIdx.x) >> 6);
  const int32_t extra = p - Q;
  const int64_t nv = n / V;
  const int64_t g = static_cast<int64_t>(blockIdx.x) * 64 + lane;
  const bool ok = g < nv;
  float s[V];
  tree_batch<Q, kHalvingFirst>(MaskedVectorLeaf<Tr, true>{bufs, g, ok}, extra, wave, s);
#pragma unroll
  for (int e = 0; e < V; ++e) lds[(wave * V + e) * 64 + lane] = s[e];
  __syncthreads();
  float t[W][V];
#pragma unroll
  for (int m = 0; m < W; ++m) {
#pragma unroll
    for (int e = 0; e < V; ++e) t[m][e] = lds[(m * V + e) * 64 + lane];
  }
#pragma unroll
  for (int d = 1; d < W; d *= 2) {
#pragma unroll
    for (int m = 0; m < W; m += 2 * d) {
#pragma unroll
      for (int e = 0; e < V; ++e) t[m][e] = t[m][e] + t[m + d][e];
    }
  }
  if (ok) {
#pragma unroll
    for (int e = 0; e < V; ++e) t[0][e] = apply_divide(t[0][e], div);
    const uint4 y = Tr::narrow(t[0]);
    const int32_t rot = store_rotation(p);
    const int32_t lo = wave * p / W, hi = (wave + 1) * p / W;
    for (int32_t k = lo; k < hi; ++k) store_vec<true>(bufs.ptr[ring_rank(rot, k, p)], g, y);
  } else if (g == nv && wave == 0) {
    for (int64_t i = nv * V; i < n; ++i) {
      float acc[1];
      tree_fold<Q, kHalvingFirst>(ElementLeaf<Tr>{bufs, i}, extra, acc);
      const float y = apply_divide(acc[0], div);
      for (int32_t r = 0; r < p; ++r) Tr::store1(bufs.ptr[r], i, y);
    }
  }
}

// ---------------------------------------------------------------------------
// Step form
// ---------------------------------------------------------------------------

enum StepOp : int32_t {
  kOpAdd = 0,      // dst = dst + src (then the step's divide)
  kOpCopy = 1,     // dst = src
  kOpPairSum = 2,  // dst = src = dst + src (then the divide): an exchange
};

// The jobs of one step, by value in the kernel arguments.
struct StepJobs {
  int64_t begin[kMaxRanks];
  int64_t end[kMaxRanks];
  int8_t dst[kMaxRanks];
  int8_t src[kMaxRanks];
};

constexpr int kStepVpt = 4;

// Job j = blockIdx.x / tiles_per_job on fp32 rows; tile 0's top lanes take
// the unaligned elements at both ends of the job's range.
template <int VPT>
__global__ __launch_bounds__(kThreads) void schedule_step_kernel(RankTable rows, StepJobs jobs,
                                                                 int32_t op,
                                                                 int32_t tiles_per_job,
                                                                 Divide div) {
  constexpr int V = 4;
  const int32_t j = static_cast<int32_t>(blockIdx.x) / tiles_per_job;
  const int32_t t = static_cast<int32_t>(blockIdx.x) - j * tiles_per_job;
  const ChunkSpan k = make_span(jobs.begin[j], jobs.end[j], V);
  if (k.s >= k.e) return;
  float *a = static_cast<float *>(rows.ptr[jobs.dst[j]]);
  float *b = static_cast<float *>(rows.ptr[jobs.src[j]]);
  const int tid = static_cast<int>(threadIdx.x);

  if (t == 0 && tid >= kThreads - 2 * (V - 1)) {
    const int lane = tid - (kThreads - 2 * (V - 1));
    const bool head = lane < V - 1;
    const int64_t i = head ? k.s + lane : k.tail_begin + (lane - (V - 1));
    if (i < (head ? k.head_end : k.e)) {
      if (op == kOpCopy) {
        a[i] = b[i];
      } else {
        const float s = apply_divide(a[i] + b[i], div);
        a[i] = s;
        if (op == kOpPairSum) b[i] = s;
      }
    }
  }

  const int64_t v0 = k.vs / V, v1 = k.ve / V;
  const int64_t base = aligned_tile_base(v0, t, int64_t(kThreads) * VPT);
  if (base >= v1) return;
  uint4 xa[VPT], xb[VPT];
  int64_t vi[VPT];
  bool ok[VPT];
#pragma unroll
  for (int u = 0; u < VPT; ++u) {
    vi[u] = base + u * kThreads + tid;
    ok[u] = vi[u] >= v0 && vi[u] < v1;
    if (ok[u]) {
      xb[u] = load_vec(b, vi[u]);
      if (op != kOpCopy) xa[u] = load_vec(a, vi[u]);
    }
  }
#pragma unroll
  for (int u = 0; u < VPT; ++u) {
    if (!ok[u]) continue;
    if (op == kOpCopy) {
      store_vec<false>(a, vi[u], xb[u]);
      continue;
    }
    float fa[4], fb[4];
    F32Traits::widen(xa[u], fa);
    F32Traits::widen(xb[u], fb);
#pragma unroll
    for (int e = 0; e < 4; ++e) fa[e] = apply_divide(fa[e] + fb[e], div);
    const uint4 y = F32Traits::narrow(fa);
    store_vec<false>(a, vi[u], y);
    if (op == kOpPairSum) store_vec<false>(b, vi[u], y);
  }
}

// ---------------------------------------------------------------------------
// Host: the schedules as lists of steps
// ---------------------------------------------------------------------------

struct Job {
  int32_t dst, src;
  int64_t begin, end;  // element range actually touched (clipped to n)
  int64_t wire;        // elements the logical message carries (padded)
};

struct Step {
  int32_t op;
  bool divide;  // this step finishes the sums: apply the average
  std::vector<Job> jobs;
};

int32_t pow2_floor(int32_t p) {
  int32_t q = 1;
  while (q * 2 <= p) q *= 2;
  return q;
}

// Extra ranks r >= q hand their buffer to r - q, and get the result back.
Step fold_in_step(int32_t p, int32_t q, int64_t n) {
  Step s{kOpAdd, false, {}};
  for (int32_t r = q; r < p; ++r) s.jobs.push_back({r - q, r, 0, n, n});
  return s;
}
Step fold_out_step(int32_t p, int32_t q, int64_t n) {
  Step s{kOpCopy, false, {}};
  for (int32_t r = q; r < p; ++r) s.jobs.push_back({r, r - q, 0, n, n});
  return s;
}

std::vector<Step> recursive_doubling_steps(int32_t p, int64_t n) {
  const int32_t q = pow2_floor(p);
  std::vector<Step> steps;
  if (q < p) steps.push_back(fold_in_step(p, q, n));
  for (int32_t d = 1; d < q; d *= 2) {
    Step s{kOpPairSum, false, {}};
    for (int32_t r = 0; r < q; ++r) {
      if ((r & d) == 0) s.jobs.push_back({r, r ^ d, 0, n, n});
    }
    steps.push_back(s);
  }
  steps.back().divide = true;
  if (q < p) steps.push_back(fold_out_step(p, q, n));
  return steps;
}

std::vector<Step> rabenseifner_steps(int32_t p, int64_t n) {
  const int32_t q = pow2_floor(p);
  const int64_t C = ceil_div(n, q);
  auto clip = [n](int64_t x) { return std::min(x, n); };
  std::vector<Step> steps;
  if (q < p) steps.push_back(fold_in_step(p, q, n));
  std::vector<int64_t> lo(q, 0);
  int64_t cnt = q;  // chunks in every rank's current range
  for (int32_t d = q / 2; d >= 1; d /= 2) {
    const int64_t half = cnt / 2;
    Step s{kOpAdd, false, {}};
    for (int32_t r = 0; r < q; ++r) {
      const int64_t keep = (r & d) ? lo[r] + half : lo[r];
      s.jobs.push_back({r, r ^ d, clip(keep * C), clip((keep + half) * C), half * C});
    }
    for (int32_t r = 0; r < q; ++r) {
      if (r & d) lo[r] += half;
    }
    cnt = half;
    steps.push_back(s);
  }
  steps.back().divide = true;
  for (int32_t d = 1; d < q; d *= 2) {
    Step s{kOpCopy, false, {}};
    for (int32_t r = 0; r < q; ++r) {
      const int64_t from = lo[r ^ d];
      s.jobs.push_back({r, r ^ d, clip(from * C), clip((from + cnt) * C), cnt * C});
    }
    for (int32_t r = 0; r < q; ++r) {
      if (r & d) lo[r] -= cnt;
    }
    cnt *= 2;
    steps.push_back(s);
  }
  if (q < p) steps.push_back(fold_out_step(p, q, n));
  return steps;
}

std::vector<Step> tree_steps(int32_t p, int64_t n) {
  int32_t K = 0;
  while ((1 << K) < p) ++K;
  std::vector<Step> steps;
  for (int32_t j = K - 1; j >= 0; --j) {
    Step s{kOpAdd, j == 0, {}};
    for (int32_t v = 0; v < (1 << j); ++v) {
      if (v + (1 << j) < p) s.jobs.push_back({v, v + (1 << j), 0, n, n});
    }
    steps.push_back(s);
  }
  for (int32_t j = 0; j < K; ++j) {
    Step s{kOpCopy, false, {}};
    for (int32_t v = 0; v < (1 << j); ++v) {
      if (v + (1 << j) < p) s.jobs.push_back({v + (1 << j), v, 0, n, n});
    }
    steps.push_back(s);
  }
  return steps;
}

std::vector<Step> build_steps(int32_t schedule, int32_t p, int64_t n) {
  if (p < 2) return {};
  if (schedule == DDP_SCHED_RECURSIVE_DOUBLING) return recursive_doubling_steps(p, n);
  if (schedule == DDP_SCHED_RABENSEIFNER) return rabenseifner_steps(p, n);
  return tree_steps(p, n);
}

// Accounting of the logical schedule (fp32 wire) and of the device traffic.
void fill_stats(ddp_comm_stats *st, const std::vector<Step> &steps, int32_t p, int64_t n,
                int32_t dtype, bool stepwise) {
  if (st == nullptr) return;
  std::vector<int64_t> sent(p, 0), recv(p, 0);
  int64_t messages = 0, total = 0, hbm = 0;
  for (const Step &s : steps) {
    for (const Job &j : s.jobs) {
      const int64_t bytes = j.wire * 4;
      const int64_t len = std::max<int64_t>(0, j.end - j.begin);
      sent[j.src] += bytes;
      recv[j.dst] += bytes;
      messages += 1;
      total += bytes;
      if (s.op == kOpPairSum) {
        sent[j.dst] += bytes;
        recv[j.src] += bytes;
        messages += 1;
        total += bytes;
        hbm += 4 * len * 4;
      } else {
        hbm += (s.op == kOpAdd ? 3 : 2) * len * 4;
      }
    }
  }
  st->steps = static_cast<int64_t>(steps.size());
  st->messages = messages;
  st->bytes_sent_per_rank = p > 0 ? *std::max_element(sent.begin(), sent.end()) : 0;
  st->bytes_recv_per_rank = p > 0 ? *std::max_element(recv.begin(), recv.end()) : 0;
  st->total_bytes = total;
  if (!stepwise || p == 1) {
    st->hbm_bytes = 2 * int64_t(p) * n * elem_bytes_of(dtype);
  } else {
    if (dtype == DDP_BF16) hbm += 2 * int64_t(p) * n * (2 + 4);
    st->hbm_bytes = hbm;
  }
}

// ---------------------------------------------------------------------------
// Host: launches
// ---------------------------------------------------------------------------

#ifndef DDPSIM_TREE_WAVES
#define DDPSIM_TREE_WAVES 1  // 16 ranks and more past the Infinity Cache: a batch per wave
#endif
#ifndef DDPSIM_TREE_NT_BYTES
#define DDPSIM_TREE_NT_BYTES (int64_t(256) << 20)  // as the ring's fused kernel
#endif
#ifndef DDPSIM_TREE_WAVES_BYTES
#define DDPSIM_TREE_WAVES_BYTES DDPSIM_TREE_NT_BYTES  // the split form above this many bytes
#endif
#ifndef DDPSIM_TREE_WAVES_SMALL_TILES
// ... and at or below this many 64-vector tiles. Against one wave per tile:
// 64 ranks of 4,096 or 65,536 elements 9.4 -> 4.1 and 11.3 -> 5.5 us per
// call; between the two regimes (64 ranks of 1 Mi elements, in the
// Infinity Cache) the split lost 20% (79 -> 95 us), 32 and 24 ranks 10-28%.
#define DDPSIM_TREE_WAVES_SMALL_TILES 512
#endif

template <typename Tr, int Q, bool kHalvingFirst>
ddp_status launch_tree_q(const RankTable &tab, int32_t p, int64_t n, const Divide &div,
                         bool nt, bool waves, hipStream_t stream, CallTimer &timer) {
  const int64_t nv = n / Tr::kVec;
  const int64_t blocks = ceil_div(nv + 1, kTreeThreads);
  if (blocks > INT32_MAX) return fail(DDP_EINVAL, "allreduce_sim: n too large");
  const dim3 grid(static_cast<uint32_t>(blocks));
  const char *what = "tree_allreduce_kernel launch";
  const int32_t bound = fold_residency(DDPSIM_TREE_WGS_PER_CU, p);
  if constexpr (Q >= 16) {
    constexpr int W = Q / 8;
    // a launch holds at most 2^32 - 1 threads; past that the one-wave form runs
    // past the Infinity Cache, or few enough tiles that a call is latency-bound
    const bool split = waves || blocks <= DDPSIM_TREE_WAVES_SMALL_TILES;
    if (split && DDPSIM_TREE_WAVES && blocks * 64 * W <= int64_t(UINT32_MAX)) {
      // the residency bound counts waves: ceil(bound / W) workgroups per CU
      const size_t lds = std::max(residency_lds(bound > 0 ? (bound + W - 1) / W : 0),
                                  size_t(W) * 64 * Tr::kVec * sizeof(float));
      return launch_lds(tree_allreduce_waves_kernel<Tr, Q, kHalvingFirst>, grid, dim3(64 * W),
                        lds, stream, timer, true, "tree_allreduce_waves_kernel launch", tab, p,
                        n, div);
    }
  }
  const size_t lds = residency_lds(bound);
  if (nt) {
    return launch_lds(tree_allreduce_kernel<Tr, Q, kHalvingFirst, true>, grid, dim3(kTreeThreads),
                      lds, stream, timer, true, what, tab, p, n, div);
  }
  return launch_lds(tree_allreduce_kernel<Tr, Q, kHalvingFirst, false>, grid, dim3(kTreeThreads),
                    lds, stream, timer, true, what, tab, p, n, div);
}

template <typename Tr, bool kHalvingFirst>
ddp_status launch_tree(const RankTable &tab, int32_t p, int64_t n, const Divide &div, bool nt,
                       bool waves, hipStream_t stream, CallTimer &timer) {
  switch (pow2_floor(p)) {
    case 1: return launch_tree_q<Tr, 1, kHalvingFirst>(tab, p, n, div, nt, waves, stream, timer);
    case 2: return launch_tree_q<Tr, 2, kHalvingFirst>(tab, p, n, div, nt, waves, stream, timer);
    case 4: return launch_tree_q<Tr, 4, kHalvingFirst>(tab, p, n, div, nt, waves, stream, timer);
    case 8: return launch_tree_q<Tr, 8, kHalvingFirst>(tab, p, n, div, nt, waves, stream, timer);
    case 16: return launch_tree_q<Tr, 16, kHalvingFirst>(tab, p, n, div, nt, waves, stream, timer);
    case 32: return launch_tree_q<Tr, 32, kHalvingFirst>(tab, p, n, div, nt, waves, stream, timer);
    default: return launch_tree_q<Tr, 64, kHalvingFirst>(tab, p, n, div, nt, waves, stream, timer);
  }
}

ddp_status launch_fused_tree(const RankTable &tab, int32_t p, int64_t n, int32_t dtype,
                             int32_t schedule, const Divide &div, hipStream_t stream,
                             CallTimer &timer) {
  const int64_t bytes = int64_t(p) * n * elem_bytes_of(dtype);
  const bool nt = bytes > DDPSIM_TREE_NT_BYTES;
  const bool waves = bytes > DDPSIM_TREE_WAVES_BYTES;
  const bool halving_first = schedule != DDP_SCHED_RECURSIVE_DOUBLING;
  if (dtype == DDP_F32) {
    return halving_first
               ? launch_tree<F32Traits, true>(tab, p, n, div, nt, waves, stream, timer)
               : launch_tree<F32Traits, false>(tab, p, n, div, nt, waves, stream, timer);
  }
  return halving_first ? launch_tree<BF16Traits, true>(tab, p, n, div, nt, waves, stream, timer)
                       : launch_tree<BF16Traits, false>(tab, p, n, div, nt, waves, stream, timer);
}

ddp_status launch_schedule_steps(const RankTable &rows, const std::vector<Step> &steps,
                                 const Divide &div, hipStream_t stream, CallTimer &timer,
                                 bool ends_call) {
  const Divide none{kNone, 1.0f, 1.0f};
  for (size_t k = 0; k < steps.size(); ++k) {
    const Step &s = steps[k];
    StepJobs jobs;
    int64_t longest = 0;
    for (size_t j = 0; j < s.jobs.size(); ++j) {
      jobs.begin[j] = s.jobs[j].begin;
      jobs.end[j] = s.jobs[j].end;
      jobs.dst[j] = static_cast<int8_t>(s.jobs[j].dst);
      jobs.src[j] = static_cast<int8_t>(s.jobs[j].src);
      longest = std::max(longest, s.jobs[j].end - s.jobs[j].begin);
    }
    // vectors of the longest job, plus one for a range that straddles, and
    // one more tile for a job that starts off the tile grid
    const int64_t vectors = longest / 4 + 1;
    const int32_t tpj = static_cast<int32_t>(
        std::max<int64_t>(1, ceil_div(vectors, int64_t(kThreads) * kStepVpt) + 1));
    const int64_t blocks = int64_t(tpj) * static_cast<int64_t>(s.jobs.size());
    if (blocks > INT32_MAX) return fail(DDP_EINVAL, "allreduce_sim: n too large");
    const bool last = ends_call && k + 1 == steps.size();
    ddp_status st = launch(schedule_step_kernel<kStepVpt>, dim3(static_cast<uint32_t>(blocks)),
                           dim3(kThreads), stream, timer, last, "schedule_step_kernel launch",
                           rows, jobs, s.op, tpj, s.divide ? div : none);
    if (st != DDP_OK) return st;
  }
  return DDP_OK;
}

bool known_schedule(int32_t s) { return s >= DDP_SCHED_RING && s <= DDP_SCHED_TREE; }

}  // namespace
}  // namespace ddpsim

using namespace ddpsim;

extern "C" size_t allreduce_sim_workspace(int32_t p, int64_t n, int32_t dtype, int32_t schedule,
                                          int32_t steps) {
  if (schedule == DDP_SCHED_RING) {
    return ring_allreduce_sim_workspace(p, n, dtype, steps ? DDP_ALGO_RING : DDP_ALGO_FUSED);
  }
  if (p < 2 || p > kMaxRanks || n <= 0 || !steps || dtype != DDP_BF16) return 0;
  return static_cast<size_t>(p) * workspace_stride_elems(n) * 4;
}

extern "C" ddp_status allreduce_sim(void *const *bufs, int32_t p, int64_t n, int32_t dtype,
                                    int32_t avg_mode, const int64_t *tokens, int32_t schedule,
                                    int32_t steps, void *workspace, size_t workspace_bytes,
                                    hipStream_t stream, ddp_comm_stats *stats) {
  clear_error();
  if (!known_schedule(schedule)) {
    return fail(DDP_EINVAL, "allreduce_sim: unknown schedule %d", schedule);
  }
  if (steps != 0 && steps != 1) return fail(DDP_EINVAL, "allreduce_sim: steps must be 0 or 1");
  if (schedule == DDP_SCHED_RING) {
    return ring_allreduce_sim(bufs, p, n, dtype, avg_mode, tokens,
                              steps ? DDP_ALGO_RING : DDP_ALGO_FUSED, workspace,
                              workspace_bytes, stream, stats);
  }
  CallTimer timer = CallTimer::take();
  Divide div;
  ddp_status s = validate_allreduce(bufs, p, n, dtype, avg_mode, tokens, &div, "allreduce_sim");
  if (s != DDP_OK) return s;
  const size_t need = allreduce_sim_workspace(p, n, dtype, schedule, steps);
  s = check_workspace("allreduce_sim", workspace, workspace_bytes, need, bufs, p,
                      n * elem_bytes_of(dtype));
  if (s != DDP_OK) return s;
  const std::vector<Step> plan = build_steps(schedule, p, n);
  fill_stats(stats, plan, p, n, dtype, steps != 0);
  if (n == 0) return DDP_OK;
  const RankTable tab = make_table(bufs, p);
  if (!steps || p == 1) return launch_fused_tree(tab, p, n, dtype, schedule, div, stream, timer);
  if (dtype == DDP_F32) return launch_schedule_steps(tab, plan, div, stream, timer, true);

  // bf16: widen into fp32 rows, run the steps there, round back once.
  const int64_t stride = workspace_stride_elems(n);
  float *ws = static_cast<float *>(workspace);
  const int32_t tpr = static_cast<int32_t>(ceil_div(ceil_div(n, 8), kThreads));
  const int64_t blocks = int64_t(tpr) * p;
  if (blocks > INT32_MAX) return fail(DDP_EINVAL, "allreduce_sim: n too large");
  const dim3 grid(static_cast<uint32_t>(blocks));
  s = launch(bf16_workspace_kernel<true>, grid, dim3(kThreads), stream, timer, false,
             "bf16_workspace_kernel launch", tab, ws, stride, n, tpr);
  if (s != DDP_OK) return s;
  RankTable rows;
  for (int32_t r = 0; r < kMaxRanks; ++r) rows.ptr[r] = r < p ? ws + r * stride : nullptr;
  s = launch_schedule_steps(rows, plan, div, stream, timer, false);
  if (s != DDP_OK) return s;
  return launch(bf16_workspace_kernel<false>, grid, dim3(kThreads), stream, timer, true,
                "bf16_workspace_kernel launch", tab, ws, stride, n, tpr);
}

extern "C" double ddp_schedule_time(int32_t schedule, int32_t p, double bytes, double alpha,
                                    double beta) {
  if (!known_schedule(schedule) || p < 1 || p > (1 << 20) || !(bytes >= 0.0) ||
      !(alpha >= 0.0) || !(beta >= 0.0)) {
    return -1.0;
  }
  if (p == 1) return 0.0;
  int32_t q = 1, k = 0, K = 0;
  while (q * 2 <= p) {
    q *= 2;
    ++k;
  }
  while ((1 << K) < p) ++K;
  const double whole = alpha + beta * bytes;  // one step moving the whole buffer
  const double extra = q < p ? 2.0 * whole : 0.0;
  switch (schedule) {
    case DDP_SCHED_RING:
      return 2.0 * (p - 1) * (alpha + beta * bytes / p);
    case DDP_SCHED_RECURSIVE_DOUBLING:
      return k * whole + extra;
    case DDP_SCHED_RABENSEIFNER:
      return 2.0 * k * alpha + 2.0 * (q - 1) / q * bytes * beta + extra;
    default:
      return 2.0 * K * whole;
  }
}

extern "C" int32_t ddp_choose_schedule(int32_t p, int64_t bytes, double alpha, double beta,
                                       uint32_t candidates) {
  clear_error();
  if (p < 1 || bytes < 0 || !(alpha >= 0.0) || !(beta >= 0.0)) {
    fail(DDP_EINVAL, "ddp_choose_schedule: bad arguments");
    return -1;
  }
  int32_t best = -1;
  double best_t = 0.0;
  for (int32_t s = DDP_SCHED_RING; s <= DDP_SCHED_TREE; ++s) {
    if (!(candidates & (1u << s))) continue;
    const double t = ddp_schedule_time(s, p, static_cast<double>(bytes), alpha, beta);
    if (best < 0 || t < best_t) {
      best = s;
      best_t = t;
    }
  }
  if (best < 0) fail(DDP_EINVAL, "ddp_choose_schedule: no known schedule among the candidates");
  return best;
}
