// internal.hpp -- shared declarations of libddpsim (host and device).
//
// Everything here is private to the library; the public surface is
// include/ddpsim.h.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "ddpsim.h"

namespace ddpsim {

constexpr int kThreads = 256;               // threads per workgroup (4 waves)
constexpr int kMaxRanks = DDP_MAX_RANKS;
constexpr int kVecBytes = 16;               // one global_load/store_dwordx4

// Rank buffers travel by value in the kernel arguments (64 x 8 = 512 bytes),
// so a workgroup reads a rank's base address with one scalar load.
struct RankTable {
  void *ptr[kMaxRanks];
};

// How a kernel applies the average to a finished fp32 sum.
//   kNone      leave the sum
//   kScale     multiply by an exact power-of-two reciprocal: x * 2^-k rounds
//              the same real number as x / 2^k, so the bits are identical
//   kDivide    one correctly rounded fp32 division
enum DivideMode : int32_t { kNone = 0, kScale = 1, kDivide = 2 };

struct Divide {
  int32_t mode;
  float divisor;
  float recip;
};

// One parameter of a bucket plan, as the flatten kernels read it from the
// plan's device table (32 bytes, fill order, all buckets back to back).
struct ParamDesc {
  int64_t bucket_offset;  // element offset of the parameter in its bucket
  int64_t numel;          // elements of the parameter
  int32_t param;          // registration index
  int32_t tile_begin;     // first flatten tile of the parameter in its bucket
  int64_t reserved;
};
static_assert(sizeof(ParamDesc) == 32, "ParamDesc layout");

constexpr int kFlattenTile = 4096;  // elements per flatten workgroup

// One parameter of a bucket as the in-place bucket all-reduce reads it
// (32 bytes): where the parameter sits in the bucket's flat index space and
// the ring chunk size of that bucket, so that element j of the parameter is
// in ring chunk (offset + j) / chunk.
struct SegDesc {
  int64_t offset;      // element offset of the parameter in its bucket
  int64_t len;         // elements of the parameter
  int64_t chunk;       // ring chunk size C = ceil(n_b / p) of the bucket
  int32_t param;       // registration index
  int32_t tile_begin;  // first tile of the parameter (plan-wide numbering)
};
static_assert(sizeof(SegDesc) == 32, "SegDesc layout");

#ifndef DDPSIM_BUCKET_NT
#define DDPSIM_BUCKET_NT 1  // non-temporal loads and stores
#endif
#ifndef DDPSIM_BUCKET_VPT
#define DDPSIM_BUCKET_VPT 1  // 16-byte vectors per thread per tile
#endif
#ifndef DDPSIM_BUCKET_MAX_WORKGROUPS
#define DDPSIM_BUCKET_MAX_WORKGROUPS 0  // 0: one workgroup per tile
#endif
#ifndef DDPSIM_BUCKET_THREADS
#define DDPSIM_BUCKET_THREADS 64  // threads per workgroup (one wave)
#endif
#ifndef DDPSIM_BUCKET_WGS_PER_CU
#define DDPSIM_BUCKET_WGS_PER_CU 11  // workgroups resident per CU (0: no bound)
#endif
constexpr int kBucketVpt = DDPSIM_BUCKET_VPT;
constexpr int kBucketThreads = DDPSIM_BUCKET_THREADS;
#ifndef DDPSIM_BUCKET_RB
#define DDPSIM_BUCKET_RB 8  // rank loads issued before their additions
#endif
constexpr int kBucketRb = DDPSIM_BUCKET_RB;
constexpr bool kBucketNt = DDPSIM_BUCKET_NT != 0;

// The in-place kernel's tile -> descriptor map is stored grouped by tile
// mod kXcds: entry for tile t at (t % kXcds) * stride + t / kXcds, stride =
// ceil(tiles / kXcds). Consecutive workgroups of a launch run on
// consecutive XCDs, so each XCD reads one contiguous eighth of the map
// instead of every cache line of it.
constexpr int32_t kXcds = 8;
__host__ __device__ constexpr int64_t tile_map_index(int64_t t, int64_t stride) {
  return (t % kXcds) * stride + t / kXcds;
}

// elements per tile for a dtype whose 16-byte vector holds `vec` elements
constexpr int64_t bucket_tile_elems(int vec) { return int64_t(kBucketThreads) * kBucketVpt * vec; }

// ---------------------------------------------------------------------------
// Host helpers (defined in host.cpp)
// ---------------------------------------------------------------------------

void clear_error();
ddp_status fail(ddp_status s, const char *fmt, ...)
    __attribute__((format(printf, 2, 3)));
ddp_status check_hip(hipError_t e, const char *what);

// Bytes per element of a ddp_dtype, or 0 if the dtype is unknown.
int elem_bytes_of(int32_t dtype);

ddp_status check_p(int32_t p, const char *what);

// Null, alignment (to `align` bytes) and pairwise overlap of p ranges of
// `bytes` each.
ddp_status check_rank_buffers(const char *what, const void *const *bufs,
                              int32_t p, int64_t bytes, int align = kVecBytes);

// True if every one of the p pointers is 16-byte aligned.
bool all_vec_aligned(const void *const *bufs, int32_t p);

// True if [a, a+na) and [b, b+nb) share a byte.
bool ranges_overlap(const void *a, int64_t na, const void *b, int64_t nb);

// Averaging divisor from the mode and the host token counts.
ddp_status make_divide(int32_t avg_mode, int32_t p, const int64_t *tokens,
                       Divide *out);

RankTable make_table(const void *const *bufs, int32_t p);

// Dynamic LDS per workgroup that leaves room for only `wgs` workgroups on
// one compute unit (0 for wgs <= 0, or when the device cannot be asked):
// the device's LDS per CU divided by wgs, in the 512-byte allocation
// granule, at most what one workgroup may take. Kernels launched with it
// never touch it; it only bounds how many of their workgroups share a CU,
// so that fewer streams compete for each memory channel's open rows.
size_t residency_lds(int32_t wgs);

// The residency bound of a fold kernel whose waves each read p ranks: `wgs`
// workgroups per CU (tuned at 8 ranks and more), scaled up for fewer ranks
// so that each CU keeps as many bytes in flight (one 1 KiB load per rank
// per wave): wgs * 8 / p, rounded up.
int32_t fold_residency(int32_t wgs, int32_t p);

// Kernels that write one loaded vector to many ranks (the fan-out copy, the
// coalesced broadcast) split the destinations of a tile over the waves of
// one workgroup: every wave loads the same source vectors (the later loads
// hit the cache; the DRAM read counters stay at one read of the source) and
// stores to its own share of the ranks, about DDPSIM_FANOUT_DESTS_PER_WAVE
// of them. Measured on one box against one wave per tile: a broadcast to 8
// ranks of 1 GiB 0.73 -> 0.80 of peak, to 64 ranks of 128 MiB 0.68 -> 0.73,
// the in-place all-gather of 8 x 1 GiB 0.73 -> 0.81, the GPT-2 parameter
// sync 0.72 -> 0.74 (0.77 with the group index made wave-uniform). Probes
// of the same pattern: 2 destinations per wave lose at 8 ranks, 16 waves
// lose at 64; separate one-wave workgroups per destination group, or one
// loading wave that shares the vectors through LDS, were slower. Group w of
// W stores ring positions [w*p/W, (w+1)*p/W) of the workgroup's rotated
// rank order.
#ifndef DDPSIM_FANOUT_DESTS_PER_WAVE
#define DDPSIM_FANOUT_DESTS_PER_WAVE 4
#endif
constexpr int32_t kMaxFanoutWaves = 8;
// Waves per workgroup for `dests` destinations per source vector: the
// smallest power of two W (at most kMaxFanoutWaves) with W * 4 >= dests.
int32_t fanout_waves(int32_t dests);

// ddp_allreduce_buckets with an optional cap on its workgroups (0: one per
// tile). Defined in bucket_allreduce.hip; the reducer uses the cap.
ddp_status allreduce_buckets(const ddp_plan *plan, int32_t first_bucket, int32_t n_buckets,
                             int32_t p, void *const *d_grad_ptrs, int32_t dtype,
                             int32_t avg_mode, const int64_t *tokens, hipStream_t stream,
                             ddp_comm_stats *stats, int32_t max_workgroups);

// p, n, dtype, averaging and rank buffers of an in-place all-reduce.
ddp_status validate_allreduce(void *const *bufs, int32_t p, int64_t n, int32_t dtype,
                              int32_t avg_mode, const int64_t *tokens, Divide *div,
                              const char *what);

// A workspace of `need` bytes (nothing to check when need is 0): present,
// large enough, 16-byte aligned, disjoint from the p rank buffers.
ddp_status check_workspace(const char *what, const void *workspace, size_t workspace_bytes,
                           size_t need, const void *const *bufs, int32_t p,
                           int64_t buf_bytes);

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Timing requested with ddp_time_next_call: the events are attached to the
// first and the last kernel dispatch of the next entry-point call made on
// this thread. take() moves the pending request into the call.
struct CallTimer {
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
  bool started = false;
  static CallTimer take();
  hipEvent_t start_event() {
    if (started) return nullptr;
    started = true;
    return start;
  }
};

// Every kernel of the library is launched through here: a plain dispatch,
// with the call's timing events attached when requested. lds_bytes of
// dynamic LDS are reserved per workgroup (the kernels that take some use
// it only to bound how many of their workgroups share a compute unit).
template <typename Kernel, typename... Args>
ddp_status launch_lds(Kernel kernel, dim3 grid, dim3 block, size_t lds_bytes,
                      hipStream_t stream, CallTimer &timer, bool last, const char *what,
                      Args... args) {
  hipExtLaunchKernelGGL(kernel, grid, block, lds_bytes, stream, timer.start_event(),
                        last ? timer.stop : nullptr, 0, args...);
  return check_hip(hipGetLastError(), what);
}

template <typename Kernel, typename... Args>
ddp_status launch(Kernel kernel, dim3 grid, dim3 block, hipStream_t stream,
                  CallTimer &timer, bool last, const char *what, Args... args) {
  return launch_lds(kernel, grid, block, 0, stream, timer, last, what, args...);
}

// ---------------------------------------------------------------------------
// Device helpers
// ---------------------------------------------------------------------------

#if defined(__HIPCC__)

__device__ __forceinline__ float apply_divide(float x, const Divide &d) {
  if (d.mode == kScale) return x * d.recip;
  if (d.mode == kDivide) return x / d.divisor;  // correctly rounded (build flag)
  return x;
}

// bf16 -> fp32 is exact: the bf16 bits are the upper half of the binary32.
__device__ __forceinline__ float bf16_lo_to_f32(uint32_t w) {
  return __uint_as_float(w << 16);
}
__device__ __forceinline__ float bf16_hi_to_f32(uint32_t w) {
  return __uint_as_float(w & 0xFFFF0000u);
}

// fp32 -> bf16, round to nearest, ties to even. Adding 0x7FFF plus the last
// kept bit carries into bit 16 exactly when the discarded half exceeds one
// half, or equals it with an odd kept part. NaN is kept quiet.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x40u;
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

// Rank buffers are device memory, but their addresses come from tables in
// memory or from other lanes, so the compiler cannot infer the address space
// and would emit flat accesses. A flat load counts against both the vector
// memory and the LDS/scalar counters and can only be waited on with a count
// of zero, so a wait for a scalar or LDS result also drains the rank loads in
// flight (the fold's eight loads were issued as four, a drain, and four).
// Every access to rank data goes through these global-space casts instead.
// The measured throughput of the fold kernels did not change (GPT-2, Llama-7B
// and p = 64 bucket launches within 0.3%), but no wait now couples the two.
template <typename T>
__device__ __forceinline__ const __attribute__((address_space(1))) T *global_ptr(const void *p) {
  return (const __attribute__((address_space(1))) T *)p;
}
template <typename T>
__device__ __forceinline__ __attribute__((address_space(1))) T *global_ptr(void *p) {
  return (__attribute__((address_space(1))) T *)p;
}

// Element traits: how a 16-byte vector of the storage type widens to fp32
// lanes and narrows back.
struct F32Traits {
  using elem = float;
  static constexpr int kVec = 4;  // elements per 16-byte vector
  __device__ static __forceinline__ void widen(const uint4 &v, float (&f)[4]) {
    f[0] = __uint_as_float(v.x);
    f[1] = __uint_as_float(v.y);
    f[2] = __uint_as_float(v.z);
    f[3] = __uint_as_float(v.w);
  }
  __device__ static __forceinline__ uint4 narrow(const float (&f)[4]) {
    return make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]),
                      __float_as_uint(f[2]), __float_as_uint(f[3]));
  }
  __device__ static __forceinline__ float load1(const void *base, int64_t i) {
    return global_ptr<float>(base)[i];
  }
  __device__ static __forceinline__ void store1(void *base, int64_t i, float v) {
    global_ptr<float>(base)[i] = v;
  }
};

struct BF16Traits {
  using elem = uint16_t;
  static constexpr int kVec = 8;
  __device__ static __forceinline__ void widen(const uint4 &v, float (&f)[8]) {
    f[0] = bf16_lo_to_f32(v.x);
    f[1] = bf16_hi_to_f32(v.x);
    f[2] = bf16_lo_to_f32(v.y);
    f[3] = bf16_hi_to_f32(v.y);
    f[4] = bf16_lo_to_f32(v.z);
    f[5] = bf16_hi_to_f32(v.z);
    f[6] = bf16_lo_to_f32(v.w);
    f[7] = bf16_hi_to_f32(v.w);
  }
  __device__ static __forceinline__ uint4 narrow(const float (&f)[8]) {
    return make_uint4(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]),
                      pack_bf16x2(f[4], f[5]), pack_bf16x2(f[6], f[7]));
  }
  __device__ static __forceinline__ float load1(const void *base, int64_t i) {
    return __uint_as_float(
        static_cast<uint32_t>(global_ptr<uint16_t>(base)[i]) << 16);
  }
  __device__ static __forceinline__ void store1(void *base, int64_t i, float v) {
    global_ptr<uint16_t>(base)[i] = static_cast<uint16_t>(f32_to_bf16_bits(v));
  }
};

// 16-byte accesses. The non-temporal forms mark the access as streaming
// (no reuse expected), which on gfx950 lets the memory system sustain more
// bandwidth when many independent streams are read and written at once.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <bool kNonTemporal = false>
__device__ __forceinline__ uint4 load_vec(const void *base, int64_t v) {
  const __attribute__((address_space(1))) u32x4 *p = global_ptr<u32x4>(base) + v;
  u32x4 x;
  if constexpr (kNonTemporal) {
    x = __builtin_nontemporal_load(p);
  } else {
    x = *p;
  }
  return make_uint4(x.x, x.y, x.z, x.w);
}

template <bool kNonTemporal>
__device__ __forceinline__ void store_vec(void *base, int64_t v, uint4 x) {
  __attribute__((address_space(1))) u32x4 *p = global_ptr<u32x4>(base) + v;
  const u32x4 y = {x.x, x.y, x.z, x.w};
  if constexpr (kNonTemporal) {
    __builtin_nontemporal_store(y, p);
  } else {
    *p = y;
  }
}

#ifndef DDPSIM_STORE_ROTATE
#define DDPSIM_STORE_ROTATE 1
#endif
// The rank a workgroup writes first when it stores one result to all p
// ranks. Rotating it with the workgroup index spreads the stores that
// neighbouring workgroups issue at the same moment over the p destination
// buffers instead of sending them all to rank 0's first (measured: about 3%
// more bandwidth on a bare 8-in / 8-out xor fold, 0.3% on the in-place
// bucket all-reduce, whose chunks already start their folds at different
// ranks; the order of the loads made no difference). Stores of one value to
// several ranks commute, so the results are unchanged.
__device__ __forceinline__ int32_t store_rotation(int32_t p, uint32_t unit = blockIdx.x) {
  return DDPSIM_STORE_ROTATE ? static_cast<int32_t>(unit % static_cast<uint32_t>(p)) : 0;
}

// Rank (first + t) mod p without a division; first < p and t < p.
__device__ __forceinline__ int32_t ring_rank(int32_t first, int32_t t,
                                             int32_t p) {
  int32_t r = first + t;
  return r >= p ? r - p : r;
}

// The element range of chunk c of an n-element buffer cut into chunks of C,
// split into a 16-byte aligned vector body and at most kVec-1 scalar
// elements on each side:
//   head  [s, head_end)      body  [vs, ve) (vector aligned)
//   tail  [tail_begin, e)
struct ChunkSpan {
  int64_t s, e, head_end, vs, ve, tail_begin;
};

// The same split for an arbitrary range [s, e).
__device__ __forceinline__ ChunkSpan make_span(int64_t s, int64_t e, int vec) {
  ChunkSpan k;
  k.s = s;
  k.e = e < s ? s : e;
  k.vs = (k.s + vec - 1) / vec * vec;
  k.ve = k.e / vec * vec;
  k.head_end = k.vs < k.e ? k.vs : k.e;
  if (k.ve < k.vs) k.ve = k.vs;           // no aligned body
  k.tail_begin = k.ve > k.head_end ? k.ve : k.head_end;
  return k;
}

// First vector of tile t of a chunk whose vector body starts at vector v0:
// tiles of tw vectors (a power of two) on a grid counted from the buffer's
// base rather than from the chunk's start, so that a tile covers whole
// 128-byte lines of a line-aligned buffer. A chunk that starts off the grid
// has a partial first tile (lanes below v0 idle) and perhaps one more tile
// than its length needs; a chunk boundary that splits a line leaves that
// line to the two chunks' tiles. (With tiles counted from each chunk's
// start, every line straddled by a tile was written in two parts by two
// workgroups: chunks 16 bytes off the grid cost the fused all-reduce 20%.)
__device__ __forceinline__ int64_t aligned_tile_base(int64_t v0, int32_t t, int64_t tw) {
  return (v0 & ~(tw - 1)) + static_cast<int64_t>(t) * tw;  // tw: a power of two
}

__device__ __forceinline__ ChunkSpan chunk_span(int64_t c, int64_t C,
                                                int64_t n, int vec) {
  const int64_t s = c * C;
  return make_span(s, s + C < n ? s + C : n, vec);
}

#endif  // __HIPCC__

}  // namespace ddpsim
