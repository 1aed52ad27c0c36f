// C ABI of the paged attention library: argument validation, split and tile
// planning, launch grouping, and the host-side page pool.  Every check runs
// before anything is enqueued; a failed call launches nothing.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cmath>
#include <cstring>
#include <new>
#include <utility>
#include <vector>

#include "paged_attn.h"
#include "pa_internal.hpp"

namespace {

using pa::kMaxLaunchStreams;
using pa::kPage;

constexpr float kLog2e = 1.4426950408889634f;

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

bool paged_any(const pa_stream* s, int32_t n) {
  for (int32_t i = 0; i < n; ++i)
    if (s[i].layout == PA_LAYOUT_PAGED && s[i].n_rows > 0) return true;
  return false;
}

// Shape checks that need no device pointer.
int check_streams_shape(const pa_stream* s, int32_t n, int32_t n_q_heads, int32_t n_kv_heads,
                        int32_t head_dim, int max_rows) {
  if (n < 0) return PA_EINVAL;
  if (n > 0 && !s) return PA_EINVAL;
  if (n_kv_heads < 1 || n_q_heads < 1 || n_q_heads % n_kv_heads != 0) return PA_EINVAL;
  if (head_dim != 128 && head_dim != 256) return PA_EUNSUPPORTED;
  std::vector<std::pair<int64_t, int64_t>> spans;
  spans.reserve((size_t)n);
  for (int32_t i = 0; i < n; ++i) {
    const pa_stream& t = s[i];
    if (t.layout != PA_LAYOUT_PAGED && t.layout != PA_LAYOUT_SLAB) return PA_EINVAL;
    if (t.reserved != 0) return PA_EINVAL;
    if (t.ctx_len < 1 || t.n_rows < 0 || t.first_pos < 0 || t.row_offset < 0) return PA_EINVAL;
    if ((int64_t)t.first_pos + t.n_rows > t.ctx_len) return PA_ERANGE;
    if (max_rows > 0 && t.n_rows > max_rows) return PA_EINVAL;
    if (t.tree_mask && t.n_rows > PA_TREE_MAX_ROWS) return PA_EINVAL;
    if (t.n_rows > 0) spans.emplace_back(t.row_offset, (int64_t)t.row_offset + t.n_rows);
  }
  std::sort(spans.begin(), spans.end());
  for (size_t i = 1; i < spans.size(); ++i)
    if (spans[i].first < spans[i - 1].second) return PA_ERANGE;
  return PA_OK;
}

int check_call(const pa_kv_cache* c, const pa_stream* s, int32_t n, int32_t n_q_heads,
               int max_rows) {
  if (!c) return PA_EINVAL;
  if (c->dtype != PA_KV_BF16 && c->dtype != PA_KV_FP8_E4M3) return PA_EINVAL;
  int rc = check_streams_shape(s, n, n_q_heads, c->n_kv_heads, c->head_dim, max_rows);
  if (rc != PA_OK) return rc;
  if (c->dtype == PA_KV_FP8_E4M3) {
    if (!(std::isfinite(c->k_scale) && c->k_scale > 0.f)) return PA_EINVAL;
    if (!(std::isfinite(c->v_scale) && c->v_scale > 0.f)) return PA_EINVAL;
  }
  if (paged_any(s, n)) {
    if (!c->k_pages || !c->v_pages || c->n_pages < 1) return PA_EINVAL;
    if (c->page_stride < (int64_t)c->n_kv_heads * kPage * c->head_dim) return PA_EINVAL;
  }
  for (int32_t i = 0; i < n; ++i) {
    const pa_stream& t = s[i];
    if (t.n_rows == 0) continue;
    if (t.layout == PA_LAYOUT_PAGED) {
      if (!t.page_table) return PA_EINVAL;
    } else {
      if (!t.k_slab || !t.v_slab) return PA_EINVAL;
      if (t.slab_cap < t.ctx_len || t.slab_cap % kPage != 0) return PA_EINVAL;
    }
  }
  return PA_OK;
}

pa::StreamArg stream_arg(const pa_kv_cache* c, const pa_stream& t) {
  pa::StreamArg a;
  std::memset(&a, 0, sizeof a);
  a.layout = t.layout;
  a.n_rows = t.n_rows;
  a.row_offset = t.row_offset;
  a.first_pos = t.first_pos;
  a.n_keys = t.first_pos + t.n_rows;
  a.page_table = t.page_table;
  a.tree_mask = t.tree_mask;
  if (t.layout == PA_LAYOUT_PAGED) {
    a.k_base = static_cast<uint8_t*>(c ? c->k_pages : nullptr);
    a.v_base = static_cast<uint8_t*>(c ? c->v_pages : nullptr);
  } else {
    a.k_base = static_cast<uint8_t*>(t.k_slab);
    a.v_base = static_cast<uint8_t*>(t.v_slab);
    a.slab_cap = t.slab_cap;
  }
  return a;
}

pa::CacheArg cache_arg(const pa_kv_cache* c) {
  pa::CacheArg a;
  a.page_stride = c->page_stride;
  a.n_pages = c->n_pages;
  a.n_kv_heads = c->n_kv_heads;
  return a;
}

int32_t splits_of(const pa_stream& t, int32_t split_keys) {
  if (t.n_rows == 0) return 0;
  const int64_t nk = (int64_t)t.first_pos + t.n_rows;
  return (int32_t)((nk + split_keys - 1) / split_keys);
}

// The decode plan: stream order is kept; streams with rows are packed into
// launch groups of at most kMaxLaunchStreams.
struct DecodePlan {
  std::vector<int32_t> splits;
  std::vector<int64_t> slot_base;
  int64_t total_slots = 0;
  std::vector<std::vector<int32_t>> groups;
};

int plan_decode(const pa_stream* s, int32_t n, int32_t n_q_heads, int32_t split_keys,
                DecodePlan& P) {
  if (split_keys < kPage || split_keys % kPage != 0) return PA_EINVAL;
  P.splits.assign((size_t)n, 0);
  P.slot_base.assign((size_t)n, 0);
  P.total_slots = 0;
  P.groups.clear();
  for (int32_t i = 0; i < n; ++i) {
    P.splits[i] = splits_of(s[i], split_keys);
    P.slot_base[i] = P.total_slots;
    P.total_slots += (int64_t)s[i].n_rows * n_q_heads * P.splits[i];
    if (s[i].n_rows == 0) continue;
    if (P.groups.empty() || (int)P.groups.back().size() == kMaxLaunchStreams)
      P.groups.emplace_back();
    P.groups.back().push_back(i);
  }
  return PA_OK;
}

size_t ws_bytes(int64_t total_slots, int32_t head_dim) {
  return align256((size_t)total_slots * head_dim * sizeof(float)) +
         align256((size_t)total_slots * 2 * sizeof(float));
}

// Row tiling of the row-tile kernel: a workgroup covers `heads` q heads of
// one kv head (a divisor of the group) and `rows` rows, its waves holding
// prefill_wg_columns (row, head) columns.
struct RowTiling {
  int32_t heads;
  int32_t rows;
};

// Prefill: the largest divisor of the group that also divides a wave's
// column count, so no wave holds a partial row and the workgroup's K/V
// tiles serve as many q heads as that allows.
RowTiling prefill_tiling(int32_t kv_dtype, int32_t head_dim, int32_t group) {
  const int32_t cols = pa::prefill_columns(kv_dtype, head_dim, false);
  int32_t hw = 1;
  for (int32_t d = 1; d <= group && d <= cols; ++d)
    if (group % d == 0 && cols % d == 0) hw = d;
  return {hw, pa::prefill_wg_columns(kv_dtype, head_dim, false) / hw};
}

// Decode streams with many columns: the largest divisor of the group that
// fits the workgroup's columns (the whole group whenever it fits), so every
// split's K/V is read by as few workgroups as possible.
RowTiling wide_tiling(int32_t kv_dtype, int32_t head_dim, int32_t group) {
  const int32_t cols = kv_dtype == PA_KV_FP8_E4M3 ? pa::verify_wg_columns(head_dim)
                                                  : pa::prefill_wg_columns(kv_dtype, head_dim, true);
  int32_t hw = 1;
  for (int32_t d = 1; d <= group && d <= cols; ++d)
    if (group % d == 0) hw = d;
  return {hw, cols / hw};
}

// A decode stream whose (row, q head) columns per kv head exceed two MFMA
// column tiles runs on the row-tile kernel in split mode, where one
// workgroup's LDS tiles feed all its columns; narrower streams keep the
// register-streaming partial kernel.  The choice depends on the stream
// alone, so its bytes do not depend on the rest of the batch.
constexpr int32_t kWideColumns = 32;
bool wide_stream(const pa_stream& t, int32_t group) {
  return (int64_t)t.n_rows * group > kWideColumns;
}

// Compute units of a gfx950 device (MI355X / MI350X).
constexpr int64_t kComputeUnits = 256;

// Consecutive splits of one (stream, kv head) that a register-streaming
// decode workgroup computes.  Once the narrow launch needs two or more rounds
// of workgroups, splits are grouped so that about one round remains: each
// workgroup then starts once and keeps its loads flowing across the split
// boundaries.  Grouping needs a split's pages to divide evenly over the four
// waves, so that every split is walked exactly as by a workgroup of its own
// (the partials do not depend on the grouping).
int32_t narrow_splits_per_wg(int64_t blocks_one_split, int32_t split_keys) {
  if (split_keys % (4 * kPage) != 0 || blocks_one_split < 2 * kComputeUnits) return 1;
  return (int32_t)((blocks_one_split + kComputeUnits - 1) / kComputeUnits);
}

// Column tiles of the register-streaming partial kernel for a launch group:
// enough for its widest narrow stream.
int32_t col_tiles_of(const pa_stream* s, const std::vector<int32_t>& grp, int32_t group) {
  int32_t mr = 0;
  for (int32_t i : grp)
    if (!wide_stream(s[i], group)) mr = std::max(mr, s[i].n_rows);
  return (group * mr + 15) / 16;
}

}  // namespace

// ---------------------------------------------------------------------------

// Host bookkeeping of a page pool: one reference count per page id (0 free).
struct pa_page_pool {
  int32_t n_pages;
  int32_t n_free;
  std::vector<int32_t> refs;
};

extern "C" {

const char* pa_status_string(int status) {
  switch (status) {
    case PA_OK: return "ok";
    case PA_EINVAL: return "invalid argument";
    case PA_ERANGE: return "rows out of range or overlapping";
    case PA_ENOSPC: return "not enough free pages";
    case PA_ETOOBIG: return "request larger than the page pool";
    case PA_EWORKSPACE: return "decode workspace missing or too small";
    case PA_EDEVICE: return "HIP launch failed";
    case PA_EUNSUPPORTED: return "unsupported head_dim";
    default: return "unknown status";
  }
}

int pa_version(void) { return (1 << 16) | 2; }

int pa_hbm_read_probe(const void* buf, size_t bytes, uint32_t* sink, void* hip_stream) {
  if (!buf || !sink || bytes == 0 || bytes % 16 != 0 || ((uintptr_t)buf & 15) ||
      bytes > (size_t)INT64_MAX)
    return PA_EINVAL;
  return pa::launch_hbm_read_probe(buf, (int64_t)bytes, sink, (hipStream_t)hip_stream) == 0
             ? PA_OK
             : PA_EDEVICE;
}

int page_pool_create(int32_t n_pages, pa_page_pool** out) {
  if (!out || n_pages < 1) return PA_EINVAL;
  *out = nullptr;
  pa_page_pool* p = new (std::nothrow) pa_page_pool;
  if (!p) return PA_EINVAL;
  try {
    p->refs.assign((size_t)n_pages, 0);
  } catch (...) {
    delete p;
    return PA_EINVAL;
  }
  p->n_pages = n_pages;
  p->n_free = n_pages;
  *out = p;
  return PA_OK;
}

void page_pool_destroy(pa_page_pool* pool) { delete pool; }

int page_pool_alloc(pa_page_pool* pool, int32_t n, int32_t* ids_out) {
  if (!pool || n < 0 || (n > 0 && !ids_out)) return PA_EINVAL;
  if (n > pool->n_pages) return PA_ETOOBIG;
  if (n > pool->n_free) return PA_ENOSPC;
  int32_t k = 0;
  for (int32_t id = 0; id < pool->n_pages && k < n; ++id)
    if (pool->refs[id] == 0) {
      pool->refs[id] = 1;
      ids_out[k++] = id;
    }
  pool->n_free -= k;
  return PA_OK;
}

namespace {
// Occurrences of each id in ids[0..n), all in [0, n_pages), else empty.
bool count_ids(const pa_page_pool* pool, const int32_t* ids, int32_t n,
               std::vector<std::pair<int32_t, int32_t>>& counts) {
  std::vector<int32_t> v(ids, ids + n);
  std::sort(v.begin(), v.end());
  counts.clear();
  for (int32_t id : v) {
    if (id < 0 || id >= pool->n_pages) return false;
    if (!counts.empty() && counts.back().first == id) ++counts.back().second;
    else counts.emplace_back(id, 1);
  }
  return true;
}
}  // namespace

int page_pool_share(pa_page_pool* pool, const int32_t* ids, int32_t n) {
  if (!pool || n < 0 || (n > 0 && !ids)) return PA_EINVAL;
  std::vector<std::pair<int32_t, int32_t>> counts;
  if (!count_ids(pool, ids, n, counts)) return PA_ERANGE;
  for (const auto& c : counts)
    if (pool->refs[c.first] == 0 || pool->refs[c.first] > INT32_MAX - c.second) return PA_ERANGE;
  for (const auto& c : counts) pool->refs[c.first] += c.second;
  return PA_OK;
}

int page_pool_free(pa_page_pool* pool, const int32_t* ids, int32_t n) {
  if (!pool || n < 0 || (n > 0 && !ids)) return PA_EINVAL;
  std::vector<std::pair<int32_t, int32_t>> counts;
  if (!count_ids(pool, ids, n, counts)) return PA_ERANGE;
  for (const auto& c : counts)
    if (pool->refs[c.first] < c.second) return PA_ERANGE;
  for (const auto& c : counts) {
    pool->refs[c.first] -= c.second;
    if (pool->refs[c.first] == 0) ++pool->n_free;
  }
  return PA_OK;
}

int32_t page_pool_refcount(const pa_page_pool* pool, int32_t id) {
  if (!pool) return PA_EINVAL;
  if (id < 0 || id >= pool->n_pages) return PA_ERANGE;
  return pool->refs[id];
}

int32_t page_pool_free_count(const pa_page_pool* pool) { return pool ? pool->n_free : PA_EINVAL; }

// ---------------------------------------------------------------------------
// Whole pages.

}  // extern "C"

namespace {

int64_t page_bytes_of(const pa_kv_cache* c) {
  return c->page_stride * (c->dtype == PA_KV_FP8_E4M3 ? 1 : 2);
}

// Checks shared by the page copies: a usable pool and ids in range.
int check_pages(const pa_kv_cache* c, const int32_t* ids, int32_t n) {
  if (!c || n < 0 || (n > 0 && !ids)) return PA_EINVAL;
  if (c->dtype != PA_KV_BF16 && c->dtype != PA_KV_FP8_E4M3) return PA_EINVAL;
  if (n == 0) return PA_OK;
  if (!c->k_pages || !c->v_pages || c->n_pages < 1 || c->page_stride < 1) return PA_EINVAL;
  if (page_bytes_of(c) % 16 != 0) return PA_EINVAL;
  for (int32_t i = 0; i < n; ++i)
    if (ids[i] < 0 || ids[i] >= c->n_pages) return PA_ERANGE;
  return PA_OK;
}

}  // namespace

extern "C" {

int page_copy(const pa_kv_cache* cache, const int32_t* src_ids, const int32_t* dst_ids,
              int32_t n, void* hip_stream) {
  int rc = check_pages(cache, src_ids, n);
  if (rc != PA_OK) return rc;
  rc = check_pages(cache, dst_ids, n);
  if (rc != PA_OK || n == 0) return rc;
  std::vector<int32_t> d(dst_ids, dst_ids + n), sv(src_ids, src_ids + n);
  std::sort(d.begin(), d.end());
  std::sort(sv.begin(), sv.end());
  for (int32_t i = 1; i < n; ++i)
    if (d[i] == d[i - 1]) return PA_ERANGE;  // two copies onto one page
  for (int32_t x : d)
    if (std::binary_search(sv.begin(), sv.end(), x)) return PA_ERANGE;  // order would matter
  for (int32_t at = 0; at < n; at += pa::kMaxCopyPairs) {
    pa::PageCopyArgs A;
    std::memset(&A, 0, sizeof A);
    A.k = static_cast<uint8_t*>(cache->k_pages);
    A.v = static_cast<uint8_t*>(cache->v_pages);
    A.page_bytes = page_bytes_of(cache);
    A.n_pairs = std::min<int32_t>(pa::kMaxCopyPairs, n - at);
    for (int32_t i = 0; i < A.n_pairs; ++i) {
      A.src[i] = src_ids[at + i];
      A.dst[i] = dst_ids[at + i];
    }
    rc = pa::launch_page_copy(A, (hipStream_t)hip_stream);
    if (rc != 0) return rc;
  }
  return PA_OK;
}

int page_save(const pa_kv_cache* cache, const int32_t* ids, int32_t n, void* host_k,
              void* host_v, void* hip_stream) {
  int rc = check_pages(cache, ids, n);
  if (rc != PA_OK || n == 0) return rc;
  if (!host_k || !host_v) return PA_EINVAL;
  const int64_t P = page_bytes_of(cache);
  for (int32_t i = 0; i < n; ++i) {
    const uint8_t* k = static_cast<const uint8_t*>(cache->k_pages) + (int64_t)ids[i] * P;
    const uint8_t* v = static_cast<const uint8_t*>(cache->v_pages) + (int64_t)ids[i] * P;
    if (hipMemcpyAsync(static_cast<uint8_t*>(host_k) + i * P, k, (size_t)P,
                       hipMemcpyDeviceToHost, (hipStream_t)hip_stream) != hipSuccess ||
        hipMemcpyAsync(static_cast<uint8_t*>(host_v) + i * P, v, (size_t)P,
                       hipMemcpyDeviceToHost, (hipStream_t)hip_stream) != hipSuccess)
      return PA_EDEVICE;
  }
  return PA_OK;
}

int page_restore(const pa_kv_cache* cache, const int32_t* ids, int32_t n, const void* host_k,
                 const void* host_v, void* hip_stream) {
  int rc = check_pages(cache, ids, n);
  if (rc != PA_OK || n == 0) return rc;
  if (!host_k || !host_v) return PA_EINVAL;
  std::vector<int32_t> d(ids, ids + n);
  std::sort(d.begin(), d.end());
  for (int32_t i = 1; i < n; ++i)
    if (d[i] == d[i - 1]) return PA_ERANGE;  // two restores onto one page
  const int64_t P = page_bytes_of(cache);
  for (int32_t i = 0; i < n; ++i) {
    uint8_t* k = static_cast<uint8_t*>(cache->k_pages) + (int64_t)ids[i] * P;
    uint8_t* v = static_cast<uint8_t*>(cache->v_pages) + (int64_t)ids[i] * P;
    if (hipMemcpyAsync(k, static_cast<const uint8_t*>(host_k) + i * P, (size_t)P,
                       hipMemcpyHostToDevice, (hipStream_t)hip_stream) != hipSuccess ||
        hipMemcpyAsync(v, static_cast<const uint8_t*>(host_v) + i * P, (size_t)P,
                       hipMemcpyHostToDevice, (hipStream_t)hip_stream) != hipSuccess)
      return PA_EDEVICE;
  }
  return PA_OK;
}

// ---------------------------------------------------------------------------

int write_kv(const pa_kv_cache* cache, const pa_stream* streams, int32_t n_streams,
             const void* k_new, const void* v_new, void* hip_stream) {
  int rc = check_call(cache, streams, n_streams, cache ? cache->n_kv_heads : 1, 0);
  if (rc != PA_OK) return rc;
  bool any = false;
  for (int32_t i = 0; i < n_streams; ++i) any |= streams[i].n_rows > 0;
  if (!any) return PA_OK;
  if (!k_new || !v_new) return PA_EINVAL;
  std::vector<int32_t> live;
  for (int32_t i = 0; i < n_streams; ++i)
    if (streams[i].n_rows > 0) live.push_back(i);
  for (size_t at = 0; at < live.size(); at += kMaxLaunchStreams) {
    pa::WriteArgs A;
    std::memset(&A, 0, sizeof A);
    A.k_new = static_cast<const uint16_t*>(k_new);
    A.v_new = static_cast<const uint16_t*>(v_new);
    A.cache = cache_arg(cache);
    A.k_scale = cache->dtype == PA_KV_FP8_E4M3 ? cache->k_scale : 1.f;
    A.v_scale = cache->dtype == PA_KV_FP8_E4M3 ? cache->v_scale : 1.f;
    int32_t rows = 0;
    for (size_t j = at; j < live.size() && j < at + kMaxLaunchStreams; ++j) {
      pa::StreamArg a = stream_arg(cache, streams[live[j]]);
      a.row_begin = rows;
      rows += a.n_rows;
      A.s[A.n_streams++] = a;
    }
    A.total_rows = rows;
    rc = pa::launch_write_kv(A, cache->dtype, cache->head_dim, (hipStream_t)hip_stream);
    if (rc != 0) return rc;
  }
  return PA_OK;
}

size_t paged_attn_decode_workspace_size(const pa_stream* streams, int32_t n_streams,
                                        int32_t n_q_heads, int32_t head_dim,
                                        int32_t split_keys) {
  if (n_streams < 0 || (n_streams > 0 && !streams) || n_q_heads < 1) return 0;
  DecodePlan P;
  if (plan_decode(streams, n_streams, n_q_heads, split_keys, P) != PA_OK) return 0;
  return ws_bytes(P.total_slots, head_dim);
}

int paged_attn_decode_plan(const pa_stream* streams, int32_t n_streams, int32_t n_q_heads,
                           int32_t n_kv_heads, int32_t head_dim, int32_t split_keys,
                           int32_t kv_dtype, int32_t* splits_out, pa_decode_plan* plan) {
  if (kv_dtype != PA_KV_BF16 && kv_dtype != PA_KV_FP8_E4M3) return PA_EINVAL;
  int rc = check_streams_shape(streams, n_streams, n_q_heads, n_kv_heads, head_dim,
                               PA_DECODE_MAX_ROWS);
  if (rc != PA_OK) return rc;
  DecodePlan P;
  rc = plan_decode(streams, n_streams, n_q_heads, split_keys, P);
  if (rc != PA_OK) return rc;
  if (splits_out)
    for (int32_t i = 0; i < n_streams; ++i) splits_out[i] = P.splits[i];
  if (plan) {
    std::memset(plan, 0, sizeof *plan);
    const int32_t group = n_q_heads / n_kv_heads;
    const RowTiling W = wide_tiling(kv_dtype, head_dim, group);
    plan->n_launch_groups = (int32_t)P.groups.size();
    for (const auto& grp : P.groups) {
      int32_t tr = 0, narrow_splits = 0, wide_items = 0;
      for (int32_t i : grp) {
        plan->total_splits += P.splits[i];
        tr += streams[i].n_rows;
        if (wide_stream(streams[i], group))
          wide_items += (streams[i].n_rows + W.rows - 1) / W.rows * P.splits[i];
        else
          narrow_splits += P.splits[i];
      }
      const int32_t ct = col_tiles_of(streams, grp, group);
      const int32_t wb = wide_items * n_kv_heads * (group / W.heads);
      const int32_t spw =
          narrow_splits_per_wg((int64_t)narrow_splits * ct * n_kv_heads, split_keys);
      int32_t narrow_items = 0;
      for (int32_t i : grp)
        if (!wide_stream(streams[i], group)) narrow_items += (P.splits[i] + spw - 1) / spw;
      plan->col_tiles = std::max(plan->col_tiles, ct);
      if (narrow_splits > 0)
        plan->narrow_splits_per_wg = std::max(plan->narrow_splits_per_wg, spw);
      plan->partial_blocks += narrow_items * ct * n_kv_heads + wb;
      plan->wide_blocks += wb;
      plan->merge_blocks += tr * n_q_heads;
    }
    plan->workspace_bytes = ws_bytes(P.total_slots, head_dim);
  }
  return PA_OK;
}

}  // extern "C"

namespace {

// The kernels of one decode launch group: the register-streaming partial
// kernel over its narrow streams, the row-tile kernel in split mode over its
// wide streams (either may have no streams), and the merge over all of them.
struct DecodeLaunch {
  pa::DecodeArgs narrow;
  pa::PrefillArgs wide;
  pa::DecodeArgs merge;
};

// Validate a decode call and build the kernel arguments of every launch
// group.  `need_q` / `need_out` say which of q and out the caller uses.
int prepare_decode(const pa_kv_cache* cache, const pa_stream* streams, int32_t n_streams,
                   const void* q, void* out, int32_t n_q_heads, float sm_scale,
                   int32_t split_keys, void* workspace, size_t workspace_bytes, bool need_q,
                   bool need_out, std::vector<DecodeLaunch>& launches) {
  launches.clear();
  int rc = check_call(cache, streams, n_streams, n_q_heads, PA_DECODE_MAX_ROWS);
  if (rc != PA_OK) return rc;
  if (need_q && !(std::isfinite(sm_scale) && sm_scale > 0.f)) return PA_EINVAL;
  DecodePlan P;
  rc = plan_decode(streams, n_streams, n_q_heads, split_keys, P);
  if (rc != PA_OK) return rc;
  if (P.groups.empty()) return PA_OK;
  if ((need_q && !q) || (need_out && !out)) return PA_EINVAL;
  const size_t need = ws_bytes(P.total_slots, cache->head_dim);
  if (!workspace || workspace_bytes < need || ((uintptr_t)workspace & 255)) return PA_EWORKSPACE;
  float* ws_o = static_cast<float*>(workspace);
  float* ws_ml = reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) +
                                          align256((size_t)P.total_slots * cache->head_dim *
                                                   sizeof(float)));
  const int32_t group = n_q_heads / cache->n_kv_heads;
  const float ks = cache->dtype == PA_KV_FP8_E4M3 ? cache->k_scale : 1.f;
  const float scale_log2 = sm_scale * ks * kLog2e;
  const float vs = cache->dtype == PA_KV_FP8_E4M3 ? cache->v_scale : 1.f;
  const RowTiling W = wide_tiling(cache->dtype, cache->head_dim, group);
  for (const auto& grp : P.groups) {
    DecodeLaunch D;
    std::memset(&D, 0, sizeof D);
    pa::DecodeArgs& A = D.merge;
    A.q = static_cast<const uint16_t*>(q);
    A.out = static_cast<uint16_t*>(out);
    A.ws_o = ws_o;
    A.ws_ml = ws_ml;
    A.cache = cache_arg(cache);
    A.n_q_heads = n_q_heads;
    A.group = group;
    A.split_keys = split_keys;
    A.scale_log2 = scale_log2;
    A.v_scale = vs;
    A.col_tiles = col_tiles_of(streams, grp, group);
    D.narrow = A;
    pa::PrefillArgs& B = D.wide;
    B.q = A.q;
    B.ws_o = ws_o;
    B.ws_ml = ws_ml;
    B.cache = A.cache;
    B.n_q_heads = n_q_heads;
    B.group = group;
    B.heads_per_wg = W.heads;
    B.rows_per_tile = W.rows;
    B.split_keys = split_keys;
    B.scale_log2 = scale_log2;
    B.v_scale = vs;
    int32_t splits = 0, rows = 0, items = 0, full = 0;
    for (int32_t i : grp) {
      pa::StreamArg a = stream_arg(cache, streams[i]);
      a.n_splits = P.splits[i];
      a.row_begin = rows;
      a.slot_base = P.slot_base[i];
      rows += a.n_rows;
      A.s[A.n_streams++] = a;
      if (wide_stream(streams[i], group)) {
        const int32_t tiles = (a.n_rows + W.rows - 1) / W.rows;
        a.block_begin = items;
        items += tiles * a.n_splits;
        a.full_begin = full;
        full += tiles * (a.n_keys / split_keys);
        a.part_begin = -1;
        B.s[B.n_streams++] = a;
      } else {
        splits += a.n_splits;
        D.narrow.s[D.narrow.n_streams++] = a;
      }
    }
    // narrow workgroup items: runs of spw consecutive splits per stream
    const int32_t spw = narrow_splits_per_wg(
        (int64_t)splits * A.col_tiles * cache->n_kv_heads, split_keys);
    int32_t items_n = 0;
    for (int32_t j = 0; j < D.narrow.n_streams; ++j) {
      D.narrow.s[j].block_begin = items_n;
      items_n += (D.narrow.s[j].n_splits + spw - 1) / spw;
    }
    D.narrow.splits_per_wg = spw;
    // Row-tile split mode runs one workgroup per CU, so the order of its
    // items decides the tail: every whole split first, then the streams'
    // shorter last splits, longest first (ties in stream order).
    {
      std::vector<int32_t> order;
      for (int32_t j = 0; j < B.n_streams; ++j)
        if (B.s[j].n_keys % split_keys != 0) order.push_back(j);
      std::stable_sort(order.begin(), order.end(), [&](int32_t x, int32_t y) {
        return B.s[x].n_keys % split_keys > B.s[y].n_keys % split_keys;
      });
      int32_t rank = full;
      for (int32_t j : order) {
        B.s[j].part_begin = rank - full;
        rank += (B.s[j].n_rows + W.rows - 1) / W.rows;
      }
    }
    A.total_rows = rows;
    D.narrow.total_items = items_n;
    B.total_tiles = items;
    B.full_tiles = full;
    launches.push_back(D);
  }
  return PA_OK;
}

// Enqueue the partial kernels of one launch group.
int launch_partials(const DecodeLaunch& D, const pa_kv_cache* cache, hipStream_t st) {
  if (D.narrow.n_streams > 0) {
    const int rc = pa::launch_decode_partials(D.narrow, cache->dtype, cache->head_dim,
                                              cache->n_kv_heads, st);
    if (rc != 0) return rc;
  }
  if (D.wide.n_streams > 0) {
    const int rc = cache->dtype == PA_KV_FP8_E4M3
                       ? pa::launch_verify(D.wide, cache->head_dim, st)
                       : pa::launch_prefill(D.wide, cache->dtype, cache->head_dim, st);
    if (rc != 0) return rc;
  }
  return 0;
}

}  // namespace

extern "C" {

int paged_attn_decode_partials(const pa_kv_cache* cache, const pa_stream* streams,
                               int32_t n_streams, const void* q, int32_t n_q_heads,
                               float sm_scale, int32_t split_keys, void* workspace,
                               size_t workspace_bytes, void* hip_stream) {
  std::vector<DecodeLaunch> L;
  int rc = prepare_decode(cache, streams, n_streams, q, nullptr, n_q_heads, sm_scale,
                          split_keys, workspace, workspace_bytes, true, false, L);
  if (rc != PA_OK) return rc;
  for (const auto& D : L) {
    rc = launch_partials(D, cache, (hipStream_t)hip_stream);
    if (rc != 0) return rc;
  }
  return PA_OK;
}

int paged_attn_decode_merge(const pa_kv_cache* cache, const pa_stream* streams,
                            int32_t n_streams, void* out, int32_t n_q_heads, int32_t split_keys,
                            const void* workspace, size_t workspace_bytes, void* hip_stream) {
  std::vector<DecodeLaunch> L;
  int rc = prepare_decode(cache, streams, n_streams, nullptr, out, n_q_heads, 1.f, split_keys,
                          const_cast<void*>(workspace), workspace_bytes, false, true, L);
  if (rc != PA_OK) return rc;
  for (const auto& D : L) {
    rc = pa::launch_decode_merge(D.merge, cache->head_dim, (hipStream_t)hip_stream);
    if (rc != 0) return rc;
  }
  return PA_OK;
}

int paged_attn_decode(const pa_kv_cache* cache, const pa_stream* streams, int32_t n_streams,
                      const void* q, void* out, int32_t n_q_heads, float sm_scale,
                      int32_t split_keys, void* workspace, size_t workspace_bytes,
                      void* hip_stream) {
  std::vector<DecodeLaunch> L;
  int rc = prepare_decode(cache, streams, n_streams, q, out, n_q_heads, sm_scale, split_keys,
                          workspace, workspace_bytes, true, true, L);
  if (rc != PA_OK) return rc;
  for (const auto& D : L) {
    // A group whose streams all stream through registers with one split
    // each needs no merge: its partial kernel writes the rows directly.
    bool direct = D.wide.n_streams == 0 && D.narrow.n_streams > 0;
    for (int32_t j = 0; direct && j < D.narrow.n_streams; ++j) direct = D.narrow.s[j].n_splits == 1;
    if (direct) {
      DecodeLaunch Dd = D;
      Dd.narrow.direct_out = 1;
      rc = launch_partials(Dd, cache, (hipStream_t)hip_stream);
      if (rc != 0) return rc;
      continue;
    }
    rc = launch_partials(D, cache, (hipStream_t)hip_stream);
    if (rc != 0) return rc;
    rc = pa::launch_decode_merge(D.merge, cache->head_dim, (hipStream_t)hip_stream);
    if (rc != 0) return rc;
  }
  return PA_OK;
}

int paged_attn_decode_noalloc(const pa_kv_cache* cache, const pa_stream* streams,
                              int32_t n_streams, const void* q, void* out, int32_t n_q_heads,
                              float sm_scale, int32_t split_keys, void* hip_stream) {
  static_assert(pa::kNoAllocScratchBytes == (size_t)PA_NOALLOC_SCRATCH_BYTES,
                "header and library agree on the scratch size");
  int rc = check_call(cache, streams, n_streams, n_q_heads, PA_DECODE_MAX_ROWS);
  if (rc != PA_OK) return rc;
  DecodePlan P;
  rc = plan_decode(streams, n_streams, n_q_heads, split_keys, P);
  if (rc != PA_OK) return rc;
  if (P.groups.empty()) return PA_OK;
  if (ws_bytes(P.total_slots, cache->head_dim) > pa::kNoAllocScratchBytes) return PA_EWORKSPACE;
  void* scratch = nullptr;
  rc = pa::noalloc_scratch(&scratch);
  if (rc != 0) return rc;
  return paged_attn_decode(cache, streams, n_streams, q, out, n_q_heads, sm_scale, split_keys,
                           scratch, pa::kNoAllocScratchBytes, hip_stream);
}

int paged_attn_prefill(const pa_kv_cache* cache, const pa_stream* streams, int32_t n_streams,
                       const void* q, void* out, int32_t n_q_heads, float sm_scale,
                       void* hip_stream) {
  int rc = check_call(cache, streams, n_streams, n_q_heads, 0);
  if (rc != PA_OK) return rc;
  if (!(std::isfinite(sm_scale) && sm_scale > 0.f)) return PA_EINVAL;
  std::vector<int32_t> live;
  for (int32_t i = 0; i < n_streams; ++i)
    if (streams[i].n_rows > 0) live.push_back(i);
  if (live.empty()) return PA_OK;
  if (!q || !out) return PA_EINVAL;
  const float ks = cache->dtype == PA_KV_FP8_E4M3 ? cache->k_scale : 1.f;
  const int32_t group = n_q_heads / cache->n_kv_heads;
  const RowTiling T = prefill_tiling(cache->dtype, cache->head_dim, group);
  for (size_t at = 0; at < live.size(); at += kMaxLaunchStreams) {
    pa::PrefillArgs A;
    std::memset(&A, 0, sizeof A);
    A.q = static_cast<const uint16_t*>(q);
    A.out = static_cast<uint16_t*>(out);
    A.cache = cache_arg(cache);
    A.n_q_heads = n_q_heads;
    A.group = group;
    A.heads_per_wg = T.heads;
    A.rows_per_tile = T.rows;
    A.scale_log2 = sm_scale * ks * kLog2e;
    A.v_scale = cache->dtype == PA_KV_FP8_E4M3 ? cache->v_scale : 1.f;
    int32_t tiles = 0;
    for (size_t j = at; j < live.size() && j < at + kMaxLaunchStreams; ++j) {
      pa::StreamArg a = stream_arg(cache, streams[live[j]]);
      a.block_begin = tiles;
      tiles += (a.n_rows + T.rows - 1) / T.rows;
      A.s[A.n_streams++] = a;
    }
    A.total_tiles = tiles;
    A.xcd_remap = ((int64_t)tiles * n_q_heads / T.heads) % 8 == 0 ? 1 : 0;
    rc = pa::launch_prefill(A, cache->dtype, cache->head_dim, (hipStream_t)hip_stream);
    if (rc != 0) return rc;
  }
  return PA_OK;
}

}  // extern "C"
