// Kernel-argument blocks shared by the host planner and the gfx950 kernels.
// Stream descriptors travel by value in the kernarg segment, so a launch
// stages nothing in device memory and can be captured in a HIP graph.
#pragma once

#include <stdint.h>

namespace pa {

constexpr int kPage = 256;            // positions per page (compile-time everywhere)
constexpr int kMaxLaunchStreams = 32; // streams per kernel launch; calls are chunked

// Row-tile kernel shape per head_dim: waves per workgroup and 16-column MFMA
// n-tiles per wave.  head_dim 256: 8 waves (two per SIMD) of 16 columns, so
// each wave fits in 256 registers and the SIMD interleaves two waves;
// head_dim 128: 4 waves of 48 columns.  Both give a workgroup 128 or 192
// columns sharing one set of K/V tiles.
// Row-tile kernel shape.  A column group is the 16 * ntiles MFMA columns
// that one wave holds, or, at head_dim 256, one producer/consumer wave pair
// (the producer runs S and the softmax, the consumer P.V).  Split mode
// (decode streams with many rows, e.g. 16 verify rows x 6 heads = 96
// columns) uses two n-tiles per pair, prefill three (fewer LDS fragment
// reads per product, 192 columns per workgroup).
constexpr bool prefill_paired(int kv, int head_dim) { return (kv == 0 || kv == 1) && head_dim >= 256; }
constexpr int prefill_waves(int head_dim) { return head_dim >= 256 ? 8 : 4; }
constexpr int prefill_ntiles(int kv, int head_dim, bool split) {
  return prefill_paired(kv, head_dim) ? (split ? 2 : 3) : head_dim >= 256 ? 1 : 3;
}
constexpr int prefill_groups(int kv, int head_dim) {
  return prefill_paired(kv, head_dim) ? prefill_waves(head_dim) / 2 : prefill_waves(head_dim);
}
// A split-mode workgroup's column count is the same for both KV dtypes, so
// a decode plan (workspace and block counts) need not know the dtype.
static_assert(prefill_groups(0, 256) * prefill_ntiles(0, 256, true) ==
                  prefill_groups(1, 256) * prefill_ntiles(1, 256, true) &&
              prefill_groups(0, 128) * prefill_ntiles(0, 128, true) ==
                  prefill_groups(1, 128) * prefill_ntiles(1, 128, true),
              "workgroup columns independent of the KV dtype");

// fp8 verify kernel (wide decode streams with fp8 KV): 16-column n-tiles per
// wave; its eight waves hold two column halves, so a workgroup covers
// 32 * verify_ntiles columns (96 at head_dim 256, 128 at 128).
constexpr int verify_ntiles(int head_dim) { return head_dim >= 256 ? 3 : 4; }

struct StreamArg {
  int32_t layout;       // 0 paged, 1 slab
  int32_t n_rows;       // query rows of the stream in this call
  int32_t row_offset;   // first row in q / out / k_new
  int32_t first_pos;    // absolute position of the first row
  int32_t n_keys;       // first_pos + n_rows: keys the last row sees
  int32_t n_splits;     // decode: ceil(n_keys / split_keys)
  int32_t block_begin;  // decode: first workgroup item of the stream in the launch; prefill: first row tile
  int32_t row_begin;    // first row of the stream in the launch's row numbering
  int32_t full_begin;   // row-tile split mode: first of the stream's whole-split items
  int32_t part_begin;   // row-tile split mode: rank of its short last split's items, or -1
  int64_t slot_base;    // decode: workspace slot of (row 0, head 0, split 0)
  const int32_t* page_table;  // paged: device page ids
  uint8_t* k_base;      // paged: pool K base; slab: slab K base
  uint8_t* v_base;      // paged: pool V base; slab: slab V base
  int64_t slab_cap;     // slab: capacity in positions (multiple of 256)
  const uint32_t* tree_mask;  // ancestor words per row, or null (causal chain)
};

struct CacheArg {
  int64_t page_stride;  // elements between pages
  int32_t n_pages;
  int32_t n_kv_heads;
};

struct DecodeArgs {
  const uint16_t* q;    // bf16 [rows][Hq][D]
  uint16_t* out;        // bf16 [rows][Hq][D]
  float* ws_o;          // [slots][D] unnormalised partial outputs
  float* ws_ml;         // [slots][2] (m in log2 units, l)
  CacheArg cache;
  int32_t n_q_heads;
  int32_t group;        // q heads per kv head
  int32_t split_keys;
  int32_t n_streams;
  int32_t total_items;  // workgroup items: runs of splits_per_wg consecutive splits of a stream
  int32_t col_tiles;    // 16-column MFMA tiles per (split, kv head)
  int32_t total_rows;   // rows in this launch (merge grid)
  int32_t splits_per_wg;  // consecutive splits one workgroup computes
  int32_t direct_out;   // 1: every stream has one split; write bf16 rows to out, no partials
  float scale_log2;     // sm_scale * k_scale * log2(e)
  float v_scale;
  StreamArg s[kMaxLaunchStreams];
};

// Row-tile kernel arguments.  Without split_keys it is prefill: each work
// item is one tile of a stream's rows over all the keys they see, written as
// normalised bf16 rows.  With split_keys > 0 it is the decode partial for
// streams with many (row, q head) columns: each work item is one (row tile,
// split) of a stream, written as (m, l, o) partials into the decode workspace.
struct PrefillArgs {
  const uint16_t* q;
  uint16_t* out;          // prefill: bf16 [rows][Hq][D]
  float* ws_o;            // split mode: [slots][D] unnormalised partial outputs
  float* ws_ml;           // split mode: [slots][2] (m in log2 units, l)
  CacheArg cache;
  int32_t n_q_heads;
  int32_t group;
  int32_t n_streams;
  int32_t total_tiles;    // work items in this launch (per head group)
  int32_t heads_per_wg;   // q heads of the group a workgroup covers (divides group)
  int32_t rows_per_tile;  // rows a workgroup covers: floor(4 * columns per wave / heads_per_wg)
  int32_t split_keys;     // 0: prefill; > 0: split-K partials of this many keys
  int32_t xcd_remap;      // 1: map blocks so each XCD runs one contiguous range
  int32_t full_tiles;     // split mode: items of whole splits (per head group)
  int32_t pad0;
  float scale_log2;
  float v_scale;
  StreamArg s[kMaxLaunchStreams];
};

struct WriteArgs {
  const uint16_t* k_new;  // bf16 [rows][Hkv][D]
  const uint16_t* v_new;
  CacheArg cache;
  int32_t n_streams;
  int32_t total_rows;
  float k_scale;
  float v_scale;
  StreamArg s[kMaxLaunchStreams];
};

constexpr int kMaxCopyPairs = 128;  // page pairs per copy launch; calls are chunked

struct PageCopyArgs {
  uint8_t* k;           // pool K base
  uint8_t* v;           // pool V base
  int64_t page_bytes;   // page_stride * element size (multiple of 16)
  int32_t n_pairs;
  int32_t pad0;
  int32_t src[kMaxCopyPairs];
  int32_t dst[kMaxCopyPairs];
};

}  // namespace pa
