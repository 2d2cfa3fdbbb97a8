// plan.cpp -- bucket assignment ("PyTorch DDP Deep Dive", Part 1 "What
// _ddp_init_helper actually does" and Part 3's DDPOptimizer reverse walk;
// "Data parallelism", section "Overlapping communication with the backward
// pass") and the plan's device descriptor table.
//
// Gradients become ready in the reverse of registration order, so the walk
// starts from the last registered parameter and the first bucket it fills is
// the one whose all-reduce can start first; that bucket has the small cap.
// A bucket is closed, before the next parameter would join it, once its
// bytes have reached its cap. The same walk over an explicit order rebuilds
// the buckets from the order in which gradients were observed to become
// ready (Part 2, the rebuild before the next forward). Coalesced broadcasts
// group tensors in list order into buckets no larger than their cap.
#include <algorithm>
#include <cstring>
#include <new>
#include <vector>

#include "internal.hpp"

using namespace ddpsim;

struct ddp_plan {
  int32_t n_params = 0;
  int32_t elem_bytes = 0;
  std::vector<int64_t> numel;                // registration order
  std::vector<int32_t> bucket_of;            // per parameter
  std::vector<int64_t> offset;               // per parameter, in elements
  std::vector<std::vector<int32_t>> members; // per bucket, fill order
  std::vector<int64_t> bucket_elems;
  std::vector<int32_t> desc_first;           // first ParamDesc of each bucket
  std::vector<int32_t> tiles;                // flatten tiles of each bucket
  std::vector<int32_t> tile_first;           // first tile-map entry of each bucket
  std::vector<ParamDesc> desc;
  // device table: the descriptors, then one int32 per flatten tile naming
  // its descriptor (relative to the bucket's first); the host copy stays
  // alive for the asynchronous upload
  std::vector<unsigned char> staged;
  void *d_table = nullptr;
  bool uploaded = false;
  // in-place bucket all-reduce: one descriptor per parameter with elements
  // and the chunk size of its bucket for seg_p ranks
  int32_t seg_p = 0;
  std::vector<SegDesc> seg;
  std::vector<int32_t> seg_first, seg_count, seg_tiles, seg_tile_first;
  std::vector<unsigned char> seg_staged;  // host copy of the device table
  size_t seg_bytes = 0;                   // the tile map starts here
  int64_t seg_map_stride = 0;             // entries per XCD group of the tile map
  void *d_seg = nullptr;
};

namespace ddpsim {

// Accessors used by flatten.hip.
bool plan_bucket_info(const ddp_plan *plan, int32_t b, int32_t *first,
                      int32_t *count, int32_t *tiles, int64_t *elems,
                      const void **table, const int32_t **tile_map, int32_t *n_params,
                      int32_t *elem_bytes, bool *uploaded) {
  if (plan == nullptr || b < 0 || b >= static_cast<int32_t>(plan->members.size())) {
    return false;
  }
  *first = plan->desc_first[b];
  *count = static_cast<int32_t>(plan->members[b].size());
  *tiles = plan->tiles[b];
  *elems = plan->bucket_elems[b];
  *table = plan->d_table;
  *tile_map = plan->d_table == nullptr
                  ? nullptr
                  : reinterpret_cast<const int32_t *>(
                        static_cast<const char *>(plan->d_table) +
                        plan->desc.size() * sizeof(ParamDesc)) +
                        plan->tile_first[b];
  *n_params = plan->n_params;
  *elem_bytes = plan->elem_bytes;
  *uploaded = plan->uploaded;
  return true;
}

int32_t plan_num_buckets(const ddp_plan *plan) {
  return plan ? static_cast<int32_t>(plan->members.size()) : 0;
}

const int32_t *plan_tile_map(const ddp_plan *plan, int64_t *stride) {
  if (plan == nullptr || plan->d_seg == nullptr) return nullptr;
  *stride = plan->seg_map_stride;
  return reinterpret_cast<const int32_t *>(static_cast<const char *>(plan->d_seg) +
                                           plan->seg_bytes);
}

bool plan_segment_info(const ddp_plan *plan, int32_t b, int32_t *first, int32_t *count,
                       int32_t *tiles, int32_t *tile_first, int64_t *elems,
                       const void **table, int32_t *seg_p, int32_t *n_params,
                       int32_t *elem_bytes) {
  if (plan == nullptr || b < 0 || b >= static_cast<int32_t>(plan->members.size())) {
    return false;
  }
  *seg_p = plan->seg_p;
  *elems = plan->bucket_elems[b];
  *n_params = plan->n_params;
  *elem_bytes = plan->elem_bytes;
  *table = plan->d_seg;
  if (plan->seg_p == 0) {
    *first = *count = *tiles = *tile_first = 0;
    return true;
  }
  *first = plan->seg_first[b];
  *count = plan->seg_count[b];
  *tiles = plan->seg_tiles[b];
  *tile_first = plan->seg_tile_first[b];
  return true;
}

// One descriptor per parameter with elements, bucket after bucket, carrying
// its offset in the bucket's flat index space and the bucket's ring chunk
// size ceil(n_b / p); each parameter is cut into tiles of bucket_tile_elems
// elements (a tile may cross ring chunks: every lane finds the chunk of its
// own elements). Tiles are numbered across the whole plan, bucket after
// bucket, so one launch can cover a run of consecutive buckets.
static bool build_segments(const ddp_plan *plan, int32_t p, std::vector<SegDesc> *seg,
                           std::vector<int32_t> *first, std::vector<int32_t> *count,
                           std::vector<int32_t> *tiles, std::vector<int32_t> *tile_first,
                           std::vector<int32_t> *tile_seg) {
  const int64_t tile_elems = bucket_tile_elems(kVecBytes / plan->elem_bytes);
  int64_t t = 0;
  for (size_t b = 0; b < plan->members.size(); ++b) {
    first->push_back(static_cast<int32_t>(seg->size()));
    tile_first->push_back(static_cast<int32_t>(t));
    const int64_t t0 = t;
    const int64_t nb = plan->bucket_elems[b];
    const int64_t C = nb > 0 ? ceil_div(nb, p) : 1;
    for (int32_t i : plan->members[b]) {
      if (plan->numel[i] == 0) continue;
      SegDesc d;
      std::memset(&d, 0, sizeof d);
      d.offset = plan->offset[i];
      d.len = plan->numel[i];
      d.chunk = C;
      d.param = i;
      d.tile_begin = static_cast<int32_t>(t);
      const int64_t nt = ceil_div(d.len, tile_elems);
      t += nt;
      if (t > INT32_MAX) return false;
      tile_seg->insert(tile_seg->end(), static_cast<size_t>(nt),
                       static_cast<int32_t>(seg->size()));
      seg->push_back(d);
    }
    count->push_back(static_cast<int32_t>(seg->size()) - first->back());
    tiles->push_back(static_cast<int32_t>(t - t0));
  }
  return true;
}

}  // namespace ddpsim

// Entries of the tile map as stored (grouped by tile mod kXcds, each group
// padded to the same length).
static int64_t map_stride(size_t tiles) { return ceil_div(static_cast<int64_t>(tiles), kXcds); }

extern "C" size_t ddp_plan_segment_bytes(const ddp_plan *plan, int32_t p) {
  if (plan == nullptr || p < 1 || p > kMaxRanks) return 0;
  std::vector<SegDesc> seg;
  std::vector<int32_t> f, c, t, tf, ts;
  if (!build_segments(plan, p, &seg, &f, &c, &t, &tf, &ts)) return 0;
  return seg.size() * sizeof(SegDesc) + map_stride(ts.size()) * kXcds * sizeof(int32_t);
}

extern "C" ddp_status ddp_plan_upload_segments(ddp_plan *plan, int32_t p, void *d_table,
                                               size_t bytes, hipStream_t stream) {
  clear_error();
  if (plan == nullptr) return fail(DDP_EINVAL, "ddp_plan_upload_segments: plan is NULL");
  ddp_status s = check_p(p, "ddp_plan_upload_segments");
  if (s != DDP_OK) return s;
  std::vector<SegDesc> seg;
  std::vector<int32_t> first, count, tiles, tile_first, tile_seg;
  if (!build_segments(plan, p, &seg, &first, &count, &tiles, &tile_first, &tile_seg)) {
    return fail(DDP_EINVAL, "ddp_plan_upload_segments: a bucket is too large");
  }
  // Device layout: the descriptors, then one int32 per tile naming its
  // descriptor, grouped by tile mod kXcds (tile_map_index). Both parts are
  // staged in one host buffer that the plan keeps alive.
  const size_t seg_bytes = seg.size() * sizeof(SegDesc);
  const int64_t stride = map_stride(tile_seg.size());
  const size_t need = seg_bytes + static_cast<size_t>(stride) * kXcds * sizeof(int32_t);
  if (need > 0) {
    if (d_table == nullptr || bytes < need) {
      return fail(DDP_EINVAL, "ddp_plan_upload_segments: needs %zu bytes of device memory",
                  need);
    }
    if (reinterpret_cast<uintptr_t>(d_table) % kVecBytes != 0) {
      return fail(DDP_EALIGN, "ddp_plan_upload_segments: table is not 16-byte aligned");
    }
  }
  std::vector<unsigned char> staged(need, 0);
  if (need > 0) {
    std::memcpy(staged.data(), seg.data(), seg_bytes);
    int32_t *map = reinterpret_cast<int32_t *>(staged.data() + seg_bytes);
    for (size_t t = 0; t < tile_seg.size(); ++t) {
      map[tile_map_index(static_cast<int64_t>(t), stride)] = tile_seg[t];
    }
  }
  plan->seg.swap(seg);
  plan->seg_first.swap(first);
  plan->seg_count.swap(count);
  plan->seg_tiles.swap(tiles);
  plan->seg_tile_first.swap(tile_first);
  plan->seg_staged.swap(staged);
  plan->seg_bytes = seg_bytes;
  plan->seg_map_stride = stride;
  if (need > 0) {
    s = check_hip(hipMemcpyAsync(d_table, plan->seg_staged.data(), need,
                                 hipMemcpyHostToDevice, stream),
                  "ddp_plan_upload_segments: hipMemcpyAsync");
    if (s != DDP_OK) {
      plan->seg_p = 0;
      return s;
    }
  }
  plan->d_seg = d_table;
  plan->seg_p = p;
  return DDP_OK;
}

namespace {

// How a walk closes buckets.
//   kGradient  close a non-empty bucket whose bytes have reached its cap,
//              before the next parameter joins (the gradient buckets; the
//              first bucket's cap is min(first, cap));
//   kCoalesce  close a non-empty bucket that the next tensor would take past
//              the cap (the coalesced broadcast's buckets).
enum CloseRule { kGradient, kCoalesce };

ddp_status build_plan(const int64_t *numel, int32_t n_params, const int32_t *walk,
                      int32_t elem_bytes, int64_t cap, int64_t first_cap, CloseRule rule,
                      const char *what, ddp_plan **out) {
  clear_error();
  if (out == nullptr) return fail(DDP_EINVAL, "%s: out is NULL", what);
  *out = nullptr;
  if (n_params < 0) return fail(DDP_EINVAL, "%s: n_params < 0", what);
  if (n_params > 0 && numel == nullptr) return fail(DDP_EINVAL, "%s: numel is NULL", what);
  if (cap < 0 || first_cap < 0) return fail(DDP_EINVAL, "%s: caps must be >= 0", what);
  for (int32_t i = 0; i < n_params; ++i) {
    if (numel[i] < 0) return fail(DDP_EINVAL, "%s: numel[%d] < 0", what, i);
  }
  std::vector<int32_t> order(n_params);
  if (walk != nullptr) {
    std::vector<char> seen(n_params, 0);
    for (int32_t k = 0; k < n_params; ++k) {
      const int32_t i = walk[k];
      if (i < 0 || i >= n_params || seen[i]) {
        return fail(DDP_EINVAL, "%s: order is not a permutation (entry %d)", what, k);
      }
      seen[i] = 1;
      order[k] = i;
    }
  } else {
    for (int32_t k = 0; k < n_params; ++k) order[k] = n_params - 1 - k;
  }
  ddp_plan *plan = new (std::nothrow) ddp_plan;
  if (plan == nullptr) return fail(DDP_EINVAL, "%s: out of host memory", what);
  plan->n_params = n_params;
  plan->elem_bytes = elem_bytes;
  plan->numel.assign(numel, numel + n_params);
  plan->bucket_of.assign(n_params, -1);
  plan->offset.assign(n_params, 0);

  const int64_t small_cap = std::min(first_cap, cap);
  int64_t open_bytes = 0;
  for (int32_t i : order) {
    const bool have_open = !plan->members.empty() && !plan->members.back().empty();
    bool close = !have_open;
    if (have_open && rule == kGradient) {
      close = open_bytes >= (plan->members.size() <= 1 ? small_cap : cap);
    } else if (have_open) {
      close = open_bytes + numel[i] * elem_bytes > cap;
    }
    if (close) {
      plan->members.emplace_back();
      plan->bucket_elems.push_back(0);
      open_bytes = 0;
    }
    const int32_t b = static_cast<int32_t>(plan->members.size()) - 1;
    plan->bucket_of[i] = b;
    plan->offset[i] = plan->bucket_elems[b];
    plan->members[b].push_back(i);
    plan->bucket_elems[b] += numel[i];
    open_bytes += numel[i] * elem_bytes;
  }

  // Device descriptors, bucket after bucket, each parameter cut into
  // flatten tiles of kFlattenTile elements, and the tile -> descriptor map.
  std::vector<int32_t> tile_desc;
  for (size_t b = 0; b < plan->members.size(); ++b) {
    plan->desc_first.push_back(static_cast<int32_t>(plan->desc.size()));
    plan->tile_first.push_back(static_cast<int32_t>(tile_desc.size()));
    int64_t tiles = 0;
    int32_t k = 0;
    for (int32_t i : plan->members[b]) {
      ParamDesc d;
      std::memset(&d, 0, sizeof d);
      d.bucket_offset = plan->offset[i];
      d.numel = numel[i];
      d.param = i;
      d.tile_begin = static_cast<int32_t>(tiles);
      const int64_t nt = ceil_div(numel[i], kFlattenTile);
      tiles += nt;
      if (tiles > INT32_MAX || tile_desc.size() + nt > size_t(INT32_MAX)) {
        delete plan;
        return fail(DDP_EINVAL, "%s: bucket %zu is too large", what, b);
      }
      tile_desc.insert(tile_desc.end(), static_cast<size_t>(nt), k);
      plan->desc.push_back(d);
      ++k;
    }
    plan->tiles.push_back(static_cast<int32_t>(tiles));
  }
  const size_t desc_bytes = plan->desc.size() * sizeof(ParamDesc);
  plan->staged.resize(desc_bytes + tile_desc.size() * sizeof(int32_t));
  // (zero-size parameters have descriptors but no tiles)
  if (desc_bytes > 0) std::memcpy(plan->staged.data(), plan->desc.data(), desc_bytes);
  if (!tile_desc.empty()) {
    std::memcpy(plan->staged.data() + desc_bytes, tile_desc.data(),
                tile_desc.size() * sizeof(int32_t));
  }
  *out = plan;
  return DDP_OK;
}

}  // namespace

extern "C" ddp_status ddp_bucket_plan(const int64_t *numel, int32_t n_params,
                                      int32_t elem_bytes, int64_t bucket_cap_bytes,
                                      int64_t first_bucket_cap_bytes, ddp_plan **out) {
  if (elem_bytes != 2 && elem_bytes != 4) {
    clear_error();
    if (out != nullptr) *out = nullptr;
    return fail(DDP_EINVAL, "ddp_bucket_plan: elem_bytes must be 2 or 4");
  }
  return build_plan(numel, n_params, nullptr, elem_bytes, bucket_cap_bytes,
                    first_bucket_cap_bytes, kGradient, "ddp_bucket_plan", out);
}

extern "C" ddp_status ddp_bucket_plan_ordered(const int64_t *numel, int32_t n_params,
                                              const int32_t *order, int32_t elem_bytes,
                                              int64_t bucket_cap_bytes,
                                              int64_t first_bucket_cap_bytes, ddp_plan **out) {
  if (elem_bytes != 2 && elem_bytes != 4) {
    clear_error();
    if (out != nullptr) *out = nullptr;
    return fail(DDP_EINVAL, "ddp_bucket_plan_ordered: elem_bytes must be 2 or 4");
  }
  if (n_params > 0 && order == nullptr) {
    clear_error();
    if (out != nullptr) *out = nullptr;
    return fail(DDP_EINVAL, "ddp_bucket_plan_ordered: order is NULL");
  }
  return build_plan(numel, n_params, order, elem_bytes, bucket_cap_bytes,
                    first_bucket_cap_bytes, kGradient, "ddp_bucket_plan_ordered", out);
}

extern "C" ddp_status ddp_coalesce_plan(const int64_t *numel, int32_t n_tensors,
                                        int32_t elem_bytes, int64_t cap_bytes, ddp_plan **out) {
  if (elem_bytes != 1 && elem_bytes != 2 && elem_bytes != 4 && elem_bytes != 8) {
    clear_error();
    if (out != nullptr) *out = nullptr;
    return fail(DDP_EINVAL, "ddp_coalesce_plan: elem_bytes must be 1, 2, 4 or 8");
  }
  std::vector<int32_t> forward(n_tensors > 0 ? n_tensors : 0);
  for (int32_t i = 0; i < n_tensors; ++i) forward[i] = i;
  return build_plan(numel, n_tensors, n_tensors > 0 ? forward.data() : nullptr, elem_bytes,
                    cap_bytes, cap_bytes, kCoalesce, "ddp_coalesce_plan", out);
}

extern "C" void ddp_plan_free(ddp_plan *plan) { delete plan; }

extern "C" int32_t ddp_plan_num_params(const ddp_plan *plan) {
  return plan ? plan->n_params : -1;
}

extern "C" int32_t ddp_plan_num_buckets(const ddp_plan *plan) {
  return plan ? static_cast<int32_t>(plan->members.size()) : -1;
}

extern "C" int64_t ddp_plan_bucket_numel(const ddp_plan *plan, int32_t b) {
  if (plan == nullptr || b < 0 || b >= static_cast<int32_t>(plan->members.size())) return -1;
  return plan->bucket_elems[b];
}

extern "C" int32_t ddp_plan_bucket_size(const ddp_plan *plan, int32_t b) {
  if (plan == nullptr || b < 0 || b >= static_cast<int32_t>(plan->members.size())) return -1;
  return static_cast<int32_t>(plan->members[b].size());
}

extern "C" ddp_status ddp_plan_bucket_params(const ddp_plan *plan, int32_t b,
                                             int32_t *idx_out) {
  clear_error();
  if (plan == nullptr || idx_out == nullptr) {
    return fail(DDP_EINVAL, "ddp_plan_bucket_params: NULL argument");
  }
  if (b < 0 || b >= static_cast<int32_t>(plan->members.size())) {
    return fail(DDP_ERANGE, "ddp_plan_bucket_params: bucket %d out of range", b);
  }
  std::copy(plan->members[b].begin(), plan->members[b].end(), idx_out);
  return DDP_OK;
}

extern "C" int32_t ddp_plan_param_bucket(const ddp_plan *plan, int32_t i) {
  if (plan == nullptr || i < 0 || i >= plan->n_params) return -1;
  return plan->bucket_of[i];
}

extern "C" int64_t ddp_plan_param_offset(const ddp_plan *plan, int32_t i) {
  if (plan == nullptr || i < 0 || i >= plan->n_params) return -1;
  return plan->offset[i];
}

extern "C" int64_t ddp_plan_param_numel(const ddp_plan *plan, int32_t i) {
  if (plan == nullptr || i < 0 || i >= plan->n_params) return -1;
  return plan->numel[i];
}

extern "C" int32_t ddp_plan_elem_bytes(const ddp_plan *plan) {
  return plan ? plan->elem_bytes : -1;
}

extern "C" size_t ddp_plan_device_bytes(const ddp_plan *plan) {
  return plan ? plan->staged.size() : 0;
}

extern "C" ddp_status ddp_plan_upload(ddp_plan *plan, void *d_table, size_t bytes,
                                      hipStream_t stream) {
  clear_error();
  if (plan == nullptr) return fail(DDP_EINVAL, "ddp_plan_upload: plan is NULL");
  const size_t need = plan->staged.size();
  if (need == 0) {
    plan->d_table = d_table;
    plan->uploaded = true;
    return DDP_OK;
  }
  if (d_table == nullptr || bytes < need) {
    return fail(DDP_EINVAL, "ddp_plan_upload: needs %zu bytes of device memory", need);
  }
  if (reinterpret_cast<uintptr_t>(d_table) % kVecBytes != 0) {
    return fail(DDP_EALIGN, "ddp_plan_upload: table is not 16-byte aligned");
  }
  ddp_status s = check_hip(
      hipMemcpyAsync(d_table, plan->staged.data(), need, hipMemcpyHostToDevice, stream),
      "ddp_plan_upload: hipMemcpyAsync");
  if (s != DDP_OK) return s;
  plan->d_table = d_table;
  plan->uploaded = true;
  return DDP_OK;
}
