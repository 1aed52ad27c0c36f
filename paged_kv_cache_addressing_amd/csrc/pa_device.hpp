// Device-side building blocks for the gfx950 kernels: vector types, the MFMA
// wrapper, exact fp8 -> bf16 conversion, and the page-tile addressing layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa_kargs.hpp"

namespace pa {

typedef __bf16 v8bf __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef __bf16 v2bf __attribute__((__vector_size__(2 * sizeof(__bf16))));
typedef float v4f __attribute__((__vector_size__(4 * sizeof(float))));
typedef uint32_t v4u __attribute__((__vector_size__(4 * sizeof(uint32_t))));
typedef uint32_t v2u __attribute__((__vector_size__(2 * sizeof(uint32_t))));

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ v4u load16(const uint8_t* p) {
  return *reinterpret_cast<const v4u*>(p);
}

// Streaming load (nontemporal: the line is not kept for reuse).  For bytes a
// kernel reads exactly once, such as decode's K/V; measured 8% faster there
// than a plain load.
__device__ __forceinline__ v4u load16_stream(const uint8_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const v4u*>(p));
}

__device__ __forceinline__ v8bf as_bf(v4u x) { return __builtin_bit_cast(v8bf, x); }

// C += A * B for one 16x16x32 bf16 tile.  Per lane: A holds row (lane % 16),
// k = 8*(lane/16) .. +7; B holds column (lane % 16), the same k run; C holds
// rows 4*(lane/16) .. +3 of column (lane % 16).
__device__ __forceinline__ v4f mfma16(v8bf a, v8bf b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Eight E4M3FN codes (bytes 0..7 of lo:hi) -> eight bf16, exactly (every
// E4M3FN value is a bf16 value); element order follows byte order.
__device__ __forceinline__ v8bf fp8x8_to_bf16(uint32_t lo, uint32_t hi) {
  v2bf p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
  v2bf p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
  v2bf p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
  v2bf p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
  v4u r;
  r[0] = __builtin_bit_cast(uint32_t, p0);
  r[1] = __builtin_bit_cast(uint32_t, p1);
  r[2] = __builtin_bit_cast(uint32_t, p2);
  r[3] = __builtin_bit_cast(uint32_t, p3);
  return as_bf(r);
}

// bf16 (RNE) of a float; gfx950 lowers this to v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint16_t f2bf(float x) {
  return __builtin_bit_cast(uint16_t, (__bf16)x);
}

// Two floats -> two bf16 (RNE) in one register: one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf2(float lo, float hi) {
  typedef float v2f __attribute__((__vector_size__(2 * sizeof(float))));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((v2f{lo, hi}), v2bf));
}

// Reductions over the four 16-lane rows of a wave (the four lane groups that
// hold the C rows of one MFMA column), the result in every row.  Two lane
// swaps (v_permlane16_swap: rows 0<->1 and 2<->3; v_permlane32_swap: the two
// halves) keep them off the LDS.  Both operand orders give the same bits, so
// every row gets the identical value.
__device__ __forceinline__ float rows4_max(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto p = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  const float m = fmaxf(__builtin_bit_cast(float, (uint32_t)p[0]),
                        __builtin_bit_cast(float, (uint32_t)p[1]));
  const uint32_t w = __builtin_bit_cast(uint32_t, m);
  const auto q = __builtin_amdgcn_permlane32_swap(w, w, false, false);
  return fmaxf(__builtin_bit_cast(float, (uint32_t)q[0]), __builtin_bit_cast(float, (uint32_t)q[1]));
}

__device__ __forceinline__ float rows4_sum(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto p = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  const float m = __builtin_bit_cast(float, (uint32_t)p[0]) + __builtin_bit_cast(float, (uint32_t)p[1]);
  const uint32_t w = __builtin_bit_cast(uint32_t, m);
  const auto q = __builtin_amdgcn_permlane32_swap(w, w, false, false);
  return __builtin_bit_cast(float, (uint32_t)q[0]) + __builtin_bit_cast(float, (uint32_t)q[1]);
}

// Keep the first `nv` 16-bit elements of an 8 x bf16 vector, zero the rest.
__device__ __forceinline__ v4u keep_first_h(v4u x, int nv) {
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    uint32_t m = (2 * w < nv ? 0x0000FFFFu : 0u) | (2 * w + 1 < nv ? 0xFFFF0000u : 0u);
    x[w] &= m;
  }
  return x;
}

// Keep the first `nv` bytes of a 16-byte vector, zero the rest.
__device__ __forceinline__ v4u keep_first_b(v4u x, int nv) {
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    int k = nv - 4 * w;
    uint32_t m = k >= 4 ? 0xFFFFFFFFu : (k <= 0 ? 0u : ((1u << (8 * k)) - 1u));
    x[w] &= m;
  }
  return x;
}

// Wait until at most N of this wave's vector-memory loads are outstanding
// (LDS-DMA loads included; they complete in issue order).
template <int N>
__device__ __forceinline__ void wait_vmem() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Workgroup barrier for LDS hand-off only: this wave's LDS operations are
// complete, then s_barrier.  Unlike __syncthreads() it does not wait for
// outstanding vector-memory loads, so LDS-DMA prefetches stay in flight
// across it (their completion is awaited explicitly with vmcnt).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// LDS-DMA through a buffer resource spanning one page tile: each lane's 16
// bytes at voff + soff land at lds_dst + 16 * lane.  The buffer form is used
// rather than the global one because the compiler counts a global LDS-DMA as
// a flat access that may retire out of order with LDS reads; while one is in
// flight it then waits for every LDS read with lgkmcnt(0), which undoes the
// fragment read-ahead.  Offsets past the tile read zeros.
typedef __attribute__((address_space(3))) void lds_void;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const uint8_t* base, int bytes) {
  // dword 3: 32-bit data format (required for untyped access), no swizzle
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base), 0, bytes, 0x00020000);
}
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t rs, int voff, int soff, v4u* lds_dst) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)lds_dst, 16, voff, soff, 0, 0);
}

// ----------------------------------------------------------------------------
// Addressing layer.  A "page tile" is 256 consecutive positions of one kv
// head: positions 256*t .. 256*t+255 of a stream.  For a paged stream the
// page id PT[t] is read once per tile (a wave-uniform scalar load) and all
// key and value addresses inside the tile are base + offset; for a slab the
// base is computed from the position.  Everything after this call is the
// same code for both layouts, so paged and slab streams do the same
// arithmetic on the same bytes.  Inside a tile (j = position - 256*t):
//   K(j, d): k + (j*D + d)*esz                          (key-major rows)
//   V(j, d): v + (((j/VB)*D + d)*VB + j%VB)*esz          (VB = 64/esz keys)
// V is kept in blocks of VB keys, dim-major inside a block: the P.V operand
// (8 consecutive keys of one dim) is one 16-byte load, and the V operand of
// a VB-key chunk is one contiguous run of D*64 bytes, so every HBM line a
// chunk touches is used whole.
// `ok` is false when the page id is out of range; the tile then points at
// page 0 so nothing outside the pool is read, and the caller poisons its
// result.
struct PageTile {
  uint8_t* k;
  uint8_t* v;
  bool ok;
};

// Keys per V block: 64 bytes of one dim.
template <int ESZ>
constexpr int v_block() { return 64 / ESZ; }

// Element offset of V(j, d) inside a tile.
template <int D, int ESZ>
__host__ __device__ __forceinline__ int v_off(int j, int d) {
  constexpr int VB = v_block<ESZ>();
  return ((j / VB) * D + d) * VB + (j % VB);
}

template <int D, int ESZ>
__device__ __forceinline__ PageTile page_tile(const StreamArg& s, const CacheArg& c, int t,
                                              int g) {
  PageTile r;
  if (s.layout == 0) {
    // Scalar load through the constant address space: tracked by lgkmcnt, so
    // it never waits on (or drains) the vector loads in flight.
    typedef const __attribute__((address_space(4))) int32_t const_i32;
    const int32_t page = ((const_i32*)s.page_table)[t];
    r.ok = (uint32_t)page < (uint32_t)c.n_pages;
    int64_t base = (int64_t)(r.ok ? page : 0) * c.page_stride + (int64_t)g * kPage * D;
    r.k = s.k_base + base * ESZ;
    r.v = s.v_base + base * ESZ;
  } else {
    r.ok = true;
    int64_t base = ((int64_t)g * s.slab_cap + (int64_t)t * kPage) * D;
    r.k = s.k_base + base * ESZ;
    r.v = s.v_base + base * ESZ;
  }
  return r;
}

// The page-tile map of one (stream, kv head), with the stream's fields held
// in registers for the whole work item: tile t of a paged stream is page
// PT[t] (read by the caller, a wave-uniform scalar load), of a slab the t-th
// run of 256 positions.  Same addresses as page_tile.
template <int D, int ESZ>
struct TileMap {
  const int32_t* pt;
  uint8_t* kb;     // K of the kv head in page 0 (paged) or at position 0 (slab)
  uint8_t* vb;
  int64_t stride;  // bytes between pages (paged) or 256-position runs (slab)
  int32_t n_pages;
  bool paged;
  __device__ __forceinline__ TileMap(const StreamArg& s, const CacheArg& c, int g) {
    paged = s.layout == 0;
    pt = s.page_table;
    n_pages = c.n_pages;
    const int64_t off = (int64_t)g * (paged ? kPage : s.slab_cap) * D * ESZ;
    kb = s.k_base + off;
    vb = s.v_base + off;
    stride = paged ? c.page_stride * ESZ : (int64_t)kPage * D * ESZ;
  }
  // Page id of tile t (paged streams; loads through the constant address
  // space, tracked by lgkmcnt, so it never waits on vector loads).
  __device__ __forceinline__ int32_t id(int t) const {
    typedef const __attribute__((address_space(4))) int32_t const_i32;
    return paged ? ((const_i32*)pt)[t] : t;
  }
  // The tile given its page id (or, for a slab, its index).
  __device__ __forceinline__ PageTile tile(int32_t idv) const {
    PageTile r;
    r.ok = !paged || (uint32_t)idv < (uint32_t)n_pages;
    const int64_t off = (int64_t)(r.ok ? idv : 0) * stride;
    r.k = kb + off;
    r.v = vb + off;
    return r;
  }
};

// Index of the stream that owns launch-local work item `x`: the last stream
// whose `begin` is <= x (streams with no work are never placed in a launch).
template <int FIELD>
__device__ __forceinline__ int find_stream(const StreamArg* s, int n, int x) {
  int si = 0;
  for (int i = 1; i < n; ++i) {
    int b = FIELD == 0 ? s[i].block_begin : s[i].row_begin;
    if (x >= b) si = i;
  }
  return si;
}

// The highest lane of the wave whose predicate holds, or 0 if none; the
// result is wave-uniform.
__device__ __forceinline__ int last_lane_where(bool p) {
  const uint64_t m = __ballot(p);
  return m ? 63 - __builtin_clzll(m) : 0;
}

// find_stream in one memory round trip, for kernels whose lookup is on the
// critical path: lane i (1 <= i < n) reads stream i's begin with a vector
// load, and the highest lane whose begin is <= x names the stream (0 if
// none).  The loop above waits on each begin before reading the next.  Needs
// the whole wave active.
template <int FIELD>
__device__ __forceinline__ int find_stream_wave(const StreamArg* s, int n, int x) {
  static_assert(kMaxLaunchStreams <= 64, "one stream per lane");
  const int lane = threadIdx.x & 63;
  const int i = lane < n ? lane : 0;
  const int b = FIELD == 0 ? s[i].block_begin : s[i].row_begin;
  return last_lane_where(lane > 0 && lane < n && x >= b);
}

// Work item of a split-mode launch (decode streams with many columns),
// workgroup L of nb: blocks [0, NH * F) are the whole splits (head group
// major, then stream, row tile, split); the rest are the streams' shorter
// last splits, longest first, all head groups of one before the next.  One
// workgroup runs per compute unit, so this order decides the launch's tail.
// hgrp = kv head * (group / heads_per_wg) + head group.  The stream lookups
// are wave-wide (one lane per stream), so the whole wave must be active.
__device__ __forceinline__ void split_item(const PrefillArgs& A, int L, int nb, int& hgrp,
                                           int& si, int& tile, int& split) {
  const int rpt = A.rows_per_tile;
  const int NH = nb / A.total_tiles;
  const int F = A.full_tiles;
  const int lane = threadIdx.x & 63;
  const int i = lane < A.n_streams ? lane : 0;
  if (L < NH * F) {
    hgrp = L / F;
    const int r = L - hgrp * F;
    // the last stream whose whole splits begin at or before r; lane i tests
    // stream i (one vector load for all streams)
    si = last_lane_where(lane > 0 && lane < A.n_streams && r >= A.s[i].full_begin);
    const int nf = A.s[si].n_keys / A.split_keys;
    const int local = r - A.s[si].full_begin;
    tile = local / nf;
    split = local - tile * nf;
  } else {
    const int j = L - NH * F;
    hgrp = j % NH;
    const int r = j / NH;
    // the stream whose short last split's row tiles hold rank r
    const int pb = A.s[i].part_begin;
    si = last_lane_where(lane < A.n_streams && pb >= 0 && r >= pb &&
                         r < pb + (A.s[i].n_rows + rpt - 1) / rpt);
    tile = r - A.s[si].part_begin;
    split = A.s[si].n_splits - 1;
  }
}

}  // namespace pa
