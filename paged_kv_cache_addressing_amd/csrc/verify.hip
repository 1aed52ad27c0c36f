// Split-K partials for decode streams with many (row, q head) columns and
// fp8-e4m3 KV, for gfx950: speculative verify rows (for example 16 rows of a
// 6-head group, 96 columns per kv head), causal or along a draft tree.
//
// Each workgroup computes the partial (m, l, o) of one split_keys-key split
// for one kv head and every column of a row tile, reading the split's K and
// V from HBM once, through the page table, one lookup per page (TensorFold
// pull request #2011, "What this changes"); the merge kernel then combines
// the splits (issue #1344, "Mechanism").  Rows may carry an ancestor table
// (pull request #1355, follow-up checks, "Indexing").  The pages' fp8 tiles
// and fp8 prompt kernel (pull request #1373, "What changes"; #2011, "Kernel
// contract") multiply fp8 operands; so does this kernel.
//
// fp8 matrix cores.  Both products run on the E4M3 MFMAs, reading the stored
// K and V codes as they are (no conversion):
//   S^T = K Q^T   v_mfma_f32_16x16x128_f8f6f4, A = 16 keys x 128 dims of K;
//   O^T += V^T P^T v_mfma_f32_32x32x64_f8f6f4, A = 32 dims x 64 keys of V.
// Q and P, which are not fp8, are each carried as two E4M3 terms, x = hi + lo
// with hi = E4M3(x) and lo = E4M3(x - hi), both rounded to nearest even:
// about 8 significant bits, bf16's precision, for two products per term.
//   * Q is scaled per column by a power of two sigma that puts max|q| below
//     256 (bf16 Q then splits exactly); the logit scale becomes c / sigma.
//   * P = 2^(s - m) is scaled by 2^4, so the weights that matter stay in
//     E4M3's normal range.  The running max m may lag the true maximum by up
//     to 4 in log2 units (p <= 2^8 then): m moves only when a logit passes
//     it by more than that.  The partial reports m - 4 as its reference
//     logit, so every term 2^(s - m_ref) is still at most 2^8.
//
// Work split.  Eight waves, two per SIMD.  A step is 64 keys (a quarter of a
// page, one fp8 V block).  SIMD s computes the logits of the step's keys
// 16s .. 16s+15 (its two waves each for half of the columns), and the P.V
// product for its D/4 dims (its two waves each for one 32-dim tile of every
// column at head_dim 256, or half of the columns at 128).  Every K and V byte
// of a step is read from LDS by one SIMD; the waves exchange P (two E4M3
// terms, 64 keys x columns) and one overflow flag per wave.
//
// Running max.  Each wave computes P(v) with the running max as it stands
// and flags the step when one of its logits passes that max by more than
// the lag.  The flags travel with P(v), so one barrier per 64 keys serves
// every hand-off:
//   check of step v-1, O^T += V(v-1)^T P(v-1)^T  |  softmax(v): P(v), flag
//   S(v+1) = K(v+1) Q^T
//   -- barrier v --
// Only when a flag is set (in the first step of a split, then in well under
// one step in a hundred on random data) do the waves exchange the step's
// column maxima, move the maxima that passed, rescale the row sums and O,
// and recompute P(v-1): two more barriers.  With a lag of 2 instead of 4,
// some column of a 96-column tile moves in about half of all steps.
//
// Loads.  Every wave issues its share of each step's DMAs into rings of four
// K and four V stages: K(v+4) and V(v+2) in step v, each given about two and
// a half steps to land; the waiting wave then passes the barrier that
// publishes them (K(v+2) and V(v) are awaited before barrier v).
//
// LDS fragment orders.  Every DMA instruction reads whole 128-byte lines
// (8 keys x 128 dims of K, or 16 dims x 64 keys of the V block).  A DMA
// that gathers 64-byte half lines instead (16 keys at once) streams about
// 16% slower on this chip.  Each lane's 16 bytes land at lane*16; the lanes
// take a row's 16-byte pieces in an XOR-swizzled order, so that the operand
// reads (one piece of 16 keys, or of 32 dims, per instruction) hit every
// bank once:
//   K: QK lane (n, a) reads pieces a and 4 + a of key 16s + n (its k-step's
//     dims 16a.. and 64 + 16a..); Q's operand bytes follow the same dims;
//   V: P.V lane (d, g) reads pieces 2g and 2g + 1 of dim d's 64 keys (keys
//     32g .. 32g + 31); P's operand bytes follow the same keys.
#include "pa_device.hpp"
#include "pa_internal.hpp"

namespace pa {

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));      // one lane's 32 fp8 codes
typedef float v4fe __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v2fe __attribute__((ext_vector_type(2)));

// C += A B on the fp8 matrix cores: E4M3FN A and B (format code 0), no
// block scales.  Lane l holds row (A) or column (B) l % 16 (16x16x128) or
// l % 32 (32x32x64) with 32 codes of the k range its lane group covers; A
// and B take the same k order byte for byte, so any permutation of k shared
// by both leaves the product unchanged.
__device__ __forceinline__ v4f mfma8_16(v8i a, v8i b, v4f c) {
  return __builtin_bit_cast(
      v4f, __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, __builtin_bit_cast(v4fe, c), 0,
                                                            0, 0, 0, 0, 0));
}
__device__ __forceinline__ v16f mfma8_32(v8i a, v8i b, v16f c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

__device__ __forceinline__ v8i join8(v4u x, v4u y) {
  return v8i{(int)x[0], (int)x[1], (int)x[2], (int)x[3], (int)y[0], (int)y[1], (int)y[2], (int)y[3]};
}

// Four floats, each split into two E4M3FN terms x = hi + lo (RNE): the hi
// codes in one dword (byte i for x_i), the lo codes in another.
__device__ __forceinline__ void split4(float x0, float x1, float x2, float x3, uint32_t& hi,
                                       uint32_t& lo) {
  // the first conversion of each dword fills its low half; the second, the
  // high half, so the initial contents do not matter (no zeroing move)
  int u0, u1;
  asm("" : "=v"(u0));
  asm("" : "=v"(u1));
  int h = __builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, u0, false);
  h = __builtin_amdgcn_cvt_pk_fp8_f32(x2, x3, h, true);
  const v2fe b0 = __builtin_amdgcn_cvt_pk_f32_fp8(h, false);
  const v2fe b1 = __builtin_amdgcn_cvt_pk_f32_fp8(h, true);
  int l = __builtin_amdgcn_cvt_pk_fp8_f32(x0 - b0[0], x1 - b0[1], u1, false);
  l = __builtin_amdgcn_cvt_pk_fp8_f32(x2 - b1[0], x3 - b1[1], l, true);
  hi = (uint32_t)h;
  lo = (uint32_t)l;
}

}  // namespace

template <int D>
__global__ __launch_bounds__(512, 1) void verify_kernel(const PrefillArgs A) {
  constexpr int BK = 64;                     // keys per step
  constexpr int NTG = 2 * verify_ntiles(D);  // 16-column n-tiles per workgroup (QK)
  constexpr int NTW = NTG / 2;               // QK n-tiles per wave (a column half)
  constexpr int CW = 16 * NTW;               // QK columns per wave
  constexpr int NCOL = 16 * NTG;             // columns per workgroup
  constexpr int KK = D / 128;                // QK k-steps
  constexpr int DS = D / 4;                  // P.V dims per SIMD
  constexpr int MTS = DS / 32;               // 32-dim P.V m-tiles per SIMD (2 or 1)
  constexpr int NPV = NCOL / 32;             // 32-column P.V n-tiles per workgroup
  constexpr int NPW = MTS == 2 ? NPV : NPV / 2;  // P.V n-tiles per wave
  constexpr int TPW = D / 128;               // K (and V) DMA fragments per wave per step
  constexpr int NK = 4, NV = 4;              // K and V ring stages
  constexpr int STG = BK * D / 16;           // 16-byte entries per K (or V) stage
  constexpr int PSL = 2 * NPV * 2 * 64;      // entries per P slot: [term][n-tile][half][lane]
  constexpr int MXS = NCOL * 4;              // floats of the maxima: [column][SIMD]
  constexpr float kPScale = 4.f;             // P carries a 2^4 scale (log2 units)
  constexpr float kLag = 4.f;                // running max lags by at most this (log2 units)
  static_assert(8 * KK * 64 == STG && (D / 16) * 64 == STG, "a stage is 1 KB fragments");
  static_assert(8 * TPW * 64 == STG, "eight waves share a stage's DMAs");
  static_assert(kPage % BK == 0, "a step never straddles two pages");
  static_assert(kPScale + kLag <= 8.f, "p <= 256 fits E4M3");
  __shared__ v4u lds[(NK + NV) * STG + 2 * PSL + (MXS + 2 * NCOL + 4 + 64) / 4];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int s = wave & 3;    // SIMD: key quarter of the S product, dim slice of P.V
  const int hh = wave >> 2;  // column half (QK); dim tile or column half (P.V)
  const int n = lane & 15;   // QK lane: column of an n-tile ...
  const int a = lane >> 4;   // ... and its lane group
  const int c32 = lane & 31; // P.V lane: column of a 32-column n-tile (or dim of V^T) ...
  const int g32 = lane >> 5; // ... and its lane group
  const int G = A.group;
  const int HW = A.heads_per_wg;
  const int rpt = A.rows_per_tile;

  int hgrp, si, tile, split;
  split_item(A, (int)blockIdx.x, (int)gridDim.x, hgrp, si, tile, split);
  const int g = hgrp / (G / HW);
  const int h0 = g * G + (hgrp % (G / HW)) * HW;
  const StreamArg& S = A.s[si];
  const int row0 = tile * rpt;
  const int rows_here = min(rpt, S.n_rows - row0);
  const int pos_first = S.first_pos + row0;
  const int pos_last = pos_first + rows_here - 1;
  const int n_keys_t = pos_last + 1;  // keys the tile's last row sees
  const int k_lo = split * A.split_keys;
  const int k_end = min(k_lo + A.split_keys, n_keys_t);
  const int v_lo = k_lo / BK;
  const int v_hi = k_end > k_lo ? (k_end + BK - 1) / BK : v_lo;
  // first key some row of the tile may not see
  const int mask_from = S.tree_mask ? S.first_pos : pos_first + 1;

  struct Col {
    int row, head, pos;
    bool ok;
  };
  // Workgroup column cl: its (row, q head), recomputed where used.
  auto col_of = [&](int cl) -> Col {
    const int rl = cl / HW;
    Col k;
    k.head = h0 + (cl - rl * HW);
    k.row = row0 + rl;
    k.ok = rl < rows_here;
    k.pos = k.ok ? S.first_pos + k.row : pos_last;
    return k;
  };
  // QK column of this lane in n-tile nt (kept opaque so none of it stays live)
  auto qcol = [&](int nt) -> int {
    int ln = n;
    asm("" : "+v"(ln));
    return CW * hh + 16 * nt + ln;
  };

  const float c = A.scale_log2;
  // Q^T operands (two E4M3 terms) of this wave's columns, and per column the
  // logit scale c / sigma and the lag threshold in raw logit units.  Q's
  // loads go out first (q_load), beside the page ids and ancestor words,
  // and are split into the operands (q_split) after the first K and V
  // DMAs, so those loads' flight overlaps the page-table lookup and the
  // tiles' flight.
  v8i qh[NTW][KK], ql[NTW][KK];
  float cc[NTW];
  // bytes 0..15 of k-step kk: dims 128kk + 16a + j; bytes 16..31: dims
  // 128kk + 64 + 16a + j (four 16-byte loads of 8 bf16 each)
  v4u qraw[NTW][KK][4];
  auto q_load = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) {
      const Col k = col_of(qcol(nt));
      const uint8_t* qp = reinterpret_cast<const uint8_t*>(A.q) +
                          ((int64_t)(S.row_offset + (k.ok ? k.row : row0)) * A.n_q_heads +
                           (k.ok ? k.head : h0)) * D * 2;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
#pragma unroll
          for (int q8 = 0; q8 < 2; ++q8)
            qraw[nt][kk][2 * hf + q8] = load16(qp + (128 * kk + 64 * hf + 16 * a + 8 * q8) * 2);
    }
  };
  auto q_split = [&]() __attribute__((always_inline)) {
#pragma unroll
  for (int nt = 0; nt < NTW; ++nt) {
    const Col k = col_of(qcol(nt));
    v4u raw[KK][4];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
#pragma unroll
      for (int j = 0; j < 4; ++j) raw[kk][j] = k.ok ? qraw[nt][kk][j] : v4u{0, 0, 0, 0};
    // element e (0, 1) of dword w (0..15) of k-step kk, as a float
    auto f32 = [&](int kk, int w, int e) {
      const uint32_t u = raw[kk][w >> 2][w & 3];
      return __builtin_bit_cast(float, e ? (u & 0xFFFF0000u) : (u << 16));
    };
    float mx = 0.f;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
#pragma unroll
      for (int w = 0; w < 16; ++w)
        mx = fmaxf(mx, fmaxf(fabsf(f32(kk, w, 0)), fabsf(f32(kk, w, 1))));
    mx = rows4_max(mx);
    int e2 = 0;
    (void)__builtin_frexpf(mx, &e2);  // mx < 2^e2 (e2 = 0 for a zero column)
    const float sigma = __builtin_ldexpf(1.f, 8 - e2);
    cc[nt] = __builtin_ldexpf(c, e2 - 8);
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      uint32_t hw[8], lw[8];
#pragma unroll
      for (int w = 0; w < 8; ++w)
        split4(f32(kk, 2 * w, 0) * sigma, f32(kk, 2 * w, 1) * sigma,
               f32(kk, 2 * w + 1, 0) * sigma, f32(kk, 2 * w + 1, 1) * sigma, hw[w], lw[w]);
      qh[nt][kk] = v8i{(int)hw[0], (int)hw[1], (int)hw[2], (int)hw[3], (int)hw[4], (int)hw[5],
                       (int)hw[6], (int)hw[7]};
      ql[nt][kk] = v8i{(int)lw[0], (int)lw[1], (int)lw[2], (int)lw[3], (int)lw[4], (int)lw[5],
                       (int)lw[6], (int)lw[7]};
    }
  }
  };

  v4u* const Kring = lds;
  v4u* const Vring = lds + NK * STG;
  v4u* const Pring = Vring + NV * STG;
  float* const Mx = reinterpret_cast<float*>(Pring + 2 * PSL);  // maxima, at the end row sums
  float* const Al = Mx + MXS;                                    // rescale factors
  uint32_t* const Anc = reinterpret_cast<uint32_t*>(Al + NCOL);  // ancestor words [column]
  uint8_t* const Fb = reinterpret_cast<uint8_t*>(Anc + NCOL);      // overflow flags [slot][wave]
  int32_t* const Pid = reinterpret_cast<int32_t*>(Fb + 16);         // page ids of the item

  typedef __attribute__((address_space(3))) v4u lds_v4u;

  // Page tiles.  The stream's fields stay in registers (TileMap), and the
  // page ids are read one page ahead: the id of the K loader's next page is
  // loaded when its current page starts, four steps before it is needed.  The
  // V loader runs two steps behind the K loader, so its page is the K
  // loader's current or previous one.  Every wave loads a share of every
  // step, so each wave sees every page id of the item.
  const TileMap<D, 1> map(S, A.cache, g);
  const int t_last = v_hi > v_lo ? (v_hi - 1) >> 2 : v_lo >> 2;  // last page of the item
  PageTile TK{}, TKprev{};
  int pk = -1;
  // The item's page ids (up to 64) are copied into LDS in the prologue: a
  // page switch inside the loop then reads LDS, not the page table.  A
  // scalar load would hold up the next lgkmcnt wait (the barrier's) for a
  // trip to memory.  The first page's id is a scalar load (the prologue's
  // tiles need it before the copy lands); an item of more than 64 pages
  // reads the rest with scalar loads.
  const int t0 = v_lo >> 2;
  auto page_id = [&](int t) -> int32_t {
    const int i = t - t0;
    if (map.paged && i < 64) return __builtin_amdgcn_readfirstlane(Pid[i]);
    return map.id(t);
  };
  auto page_k = [&](int v) -> const PageTile& {
    const int t = v >> 2;
    if (t != pk) {
      const int32_t idv = pk < 0 ? map.id(t) : page_id(t);
      TKprev = TK;
      TK = map.tile(idv);
      pk = t;
    }
    return TK;
  };
  auto page_v = [&](int v) -> const PageTile& { return (v >> 2) == pk ? TK : TKprev; };
  // Each DMA instruction moves one 1 KB fragment of whole 128-byte lines:
  //   K fragment F = kb * KK + h: keys 8kb .. 8kb+7 of the step, dims
  //     128h .. 128h+127; lane l takes key l / 8, 16-byte piece
  //     (l % 8) ^ kswz(l / 8, kb) of the key's 128 bytes;
  //   V fragment G: dims 16G .. 16G+15 (each a 64-byte row of 64 keys); lane
  //     l takes dim l / 4, piece (l % 4) ^ vswz(l / 4).
  // A lane's 16 bytes land at lane*16 in the fragment, so the XOR moves the
  // pieces of a row apart across the LDS banks: the operand reads below
  // (16 keys or 32 dims at the same piece) then meet no bank conflict.
  auto kswz = [](int kl, int kb) { return (kl >> 1) + 4 * (kb & 1); };
  auto vswz = [](int dl) { return (dl >> 2) & 3; };
  auto dma_k = [&](int v) {
    const PageTile& T = page_k(v);
    const auto rs = tile_rsrc(T.k, kPage * D);
    v4u* dst = Kring + ((v - v_lo) & (NK - 1)) * STG;
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      const int f = wave * TPW + i, kb = f / KK, h = f % KK, kl = lane >> 3;
      const int piece = (lane & 7) ^ kswz(kl, kb);
      dma16(rs, (8 * kb + kl) * D + 128 * h + 16 * piece, (v & 3) * BK * D, dst + f * 64);
    }
  };
  auto dma_v = [&](int v) {
    const PageTile& T = page_v(v);
    const auto rs = tile_rsrc(T.v, kPage * D);
    v4u* dst = Vring + ((v - v_lo) & (NV - 1)) * STG;
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      const int f = wave * TPW + i, dl = lane >> 2;
      const int piece = (lane & 3) ^ vswz(dl);
      dma16(rs, (16 * f + dl) * 64 + 16 * piece, (v & 3) * D * 64, dst + f * 64);
    }
  };
  // Operand read offsets (16-byte entries within a stage).  QK: lane (n, a)
  // reads key 16s + n, pieces a and 4 + a of k-step kk: fragment
  // (2s + n / 8) * KK + kk, slot (n % 8) * 8 + (piece ^ kswz).  P.V: lane
  // (d, g) reads dim DS*s + 32*mt + d, pieces 2g and 2g + 1: fragment
  // (DS*s + 32*mt + d) / 16, slot (d % 16) * 4 + (piece ^ vswz).  The second
  // piece's slot is the first's with one bit flipped (4 + a = a ^ 4 and
  // 2g + 1 = 2g ^ 1 commute with the XOR).
  const int k_rd = ((2 * s + (n >> 3)) * KK) * 64 + (n & 7) * 8 + (a ^ kswz(n & 7, n >> 3));
  const int v_rd = ((DS * s + 32 * (MTS == 2 ? hh : 0) + c32) >> 4) * 64 + (c32 & 15) * 4 +
                   ((2 * g32) ^ vswz(c32 & 15));

  // P.V accumulators: n-tile j of this wave is workgroup n-tile n0_w + j;
  // lane (c, grp) holds rows (dims) 8q + 4grp + r of column c at index 4q + r.
  const int mt_w = MTS == 2 ? hh : 0;        // this wave's P.V dim tile
  const int n0_w = MTS == 2 ? 0 : hh * NPW;  // its first P.V n-tile
  v16f o[NPW];  // zeroed after the Q operands are built
  // Per column: the exponent offset mc (log2 units, the same in every wave of
  // the column; -FLT_MAX until the column has seen a key), so that
  // p = 2^(s*cc - mc); the row-sum partial; the last step's row-sum terms.
  // mc is the running max (in log2 units) less the scale of P (kPScale); it
  // moves when some p = 2^(s*cc - mc) would exceed 2^(kPScale + kLag).
  constexpr float kNoMax = -3.40282347e38f;
  float mc[NTW], l_part[NTW], lp[NTW];
#pragma unroll
  for (int nt = 0; nt < NTW; ++nt) {
    mc[nt] = kNoMax;
    l_part[nt] = 0.f;
    lp[nt] = 0.f;
  }

  // Scheduling groups (__builtin_amdgcn_sched_group_barrier masks).
  constexpr int kMfma = 0x008, kValu = 0x002, kDsRead = 0x100;

  // S(u) = K(u) Q^T for this SIMD's 16 keys, then, in the steps that reach a
  // row's own keys or the stream's end, the mask.
  auto qk = [&](int u, v4f (&Sx)[NTW]) __attribute__((always_inline)) {
    const lds_v4u* Lk = (const lds_v4u*)(Kring + ((u - v_lo) & (NK - 1)) * STG);
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) Sx[nt] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      const v8i ka = join8(Lk[k_rd + kk * 64], Lk[(k_rd ^ 4) + kk * 64]);
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt) {
        Sx[nt] = mfma8_16(ka, qh[nt][kk], Sx[nt]);
        Sx[nt] = mfma8_16(ka, ql[nt][kk], Sx[nt]);
      }
    }
    if (u * BK + BK - 1 >= mask_from) {
      // kept a branch (the empty volatile asm cannot be speculated): the
      // selects would otherwise run on every step
      asm volatile("");
      // lane (n, a) holds keys 16s + 4a + i of the step for its column
      const int kabs0 = u * BK + 16 * s + 4 * a;
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt) {
        const Col k = col_of(qcol(nt));
        const uint32_t anc = Anc[qcol(nt)];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int kabs = kabs0 + i, rel = kabs - S.first_pos;
          const bool anc_ok = (rel < 0) | (((anc >> (rel & 31)) & 1u) != 0u);
          const bool vis = (kabs <= k.pos) & anc_ok;
          Sx[nt][i] = vis ? Sx[nt][i] : -INFINITY;
        }
      }
    }
  };

  // Softmax of step v with the running max as it stands: P(v) as two E4M3
  // terms into P slot (v & 1), the row-sum terms lp, and (when `flag`) this
  // wave's overflow flag: some logit of its keys above the running max by
  // more than the lag, so that P(v) may not fit the scale.
  const int p_lane = n * 4 + a;  // dword of a P entry that this lane writes
  auto soft = [&](int v, const v4f (&Sx)[NTW], bool flag) __attribute__((always_inline)) {
    v4u* pd = Pring + ((v - v_lo) & 1) * PSL;
    bool ov = false;
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) {
      float t[4], p[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        t[i] = __builtin_fmaf(Sx[nt][i], cc[nt], -mc[nt]);
        p[i] = __builtin_amdgcn_exp2f(t[i]);
      }
      lp[nt] = (p[0] + p[1]) + (p[2] + p[3]);
      uint32_t hi, lo;
      split4(p[0], p[1], p[2], p[3], hi, lo);
      // key 16s + 4a + i = 32 gp + 16 bp + 4a + i: dword a of the P.V operand
      // entry (half bp) of lane (column % 32, gp).  The wave's column base
      // cb = CW hh + 16 nt is a multiple of 16, so column cb + n stays in
      // 32-column tile cb / 32 at lane (cb % 32) + n: a wave-uniform entry
      // plus the lane's dword n * 4 + a.
      const int cb = CW * hh + 16 * nt;
      const int eu = ((cb >> 5) * 2 + (s & 1)) * 64 + (cb & 31) + 32 * (s >> 1);
      uint32_t* dh = reinterpret_cast<uint32_t*>(pd + eu) + p_lane;
      dh[0] = hi;
      dh[NPV * 2 * 64 * 4] = lo;  // the lo term's entries follow the hi term's
      ov |= fmaxf(fmaxf(t[0], t[1]), fmaxf(t[2], t[3])) > kPScale + kLag;
    }
    if (flag) {
      const bool any = __any(ov);
      if (lane == 0) Fb[((v - v_lo) & 1) * 8 + wave] = any ? 1 : 0;
    }
  };

  // Step u overflowed in some wave: every wave takes this path (they all
  // read the same flags).  The column maxima of the step are exchanged; a
  // column whose maximum passed its running max by more than the lag moves
  // it there; the row sums and (after the second barrier) the P.V
  // accumulators are rescaled, and P(u) and its row-sum terms recomputed.
  auto redo = [&](int u, const v4f (&Sx)[NTW]) __attribute__((always_inline)) {
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) {
      const float m4 = fmaxf(fmaxf(Sx[nt][0], Sx[nt][1]), fmaxf(Sx[nt][2], Sx[nt][3]));
      const float m = rows4_max(m4);
      if (a == 0) Mx[qcol(nt) * 4 + s] = m;
    }
    lds_barrier();  // publishes the maxima
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) {
      const v4f m4 = *reinterpret_cast<const v4f*>(Mx + qcol(nt) * 4);
      const float m = fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3]));
      float alpha = 1.f;
      if (__builtin_fmaf(m, cc[nt], -mc[nt]) > kPScale + kLag) {
        const float mn = m * cc[nt] - kPScale;
        alpha = __builtin_amdgcn_exp2f(mc[nt] - mn);  // 0 for a column's first keys
        mc[nt] = mn;
      }
      l_part[nt] *= alpha;
      if (s == 0 && a == 0) Al[qcol(nt)] = alpha;
    }
    soft(u, Sx, false);
    lds_barrier();  // publishes P(u) and the rescale factors
#pragma unroll
    for (int j = 0; j < NPW; ++j) o[j] *= Al[32 * (n0_w + j) + c32];
  };

  // Before the P.V of step u: the overflow flags of step u (published by
  // barrier u), the slow path when any is set, then the row sums.
  auto check = [&](int u, const v4f (&Sx)[NTW]) __attribute__((always_inline)) {
    const uint64_t f = *reinterpret_cast<const uint64_t*>(Fb + ((u - v_lo) & 1) * 8);
    const uint32_t any = __builtin_amdgcn_readfirstlane((uint32_t)f | (uint32_t)(f >> 32));
    if (any != 0) redo(u, Sx);
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) l_part[nt] += lp[nt];
  };

  // P.V of step u (O^T += V(u)^T P(u)^T over its 64 keys for this wave's
  // dims and columns): pv_prep reads the V operand, pv_body multiplies.
  auto pv_prep = [&](int u, bool tail) -> v8i {
    const lds_v4u* Lv = (const lds_v4u*)(Vring + ((u - v_lo) & (NV - 1)) * STG);
    v4u x0 = Lv[v_rd], x1 = Lv[v_rd ^ 1];
    if (tail) {
      // the stream's last step may run past its last key: those values
      // (unwritten slots, possibly NaN codes) become zeros
      const int k0 = u * BK + 32 * g32;
      x0 = keep_first_b(x0, n_keys_t - k0);
      x1 = keep_first_b(x1, n_keys_t - k0 - 16);
    }
    return join8(x0, x1);
  };
  auto pv_body = [&](int u, const v8i& va) {
    const lds_v4u* Lp = (const lds_v4u*)(Pring + ((u - v_lo) & 1) * PSL + lane);
#pragma unroll
    for (int j = 0; j < NPW; ++j) {
      const int N = n0_w + j;
      const v8i ph = join8(Lp[((0 * NPV + N) * 2 + 0) * 64], Lp[((0 * NPV + N) * 2 + 1) * 64]);
      const v8i pl = join8(Lp[((1 * NPV + N) * 2 + 0) * 64], Lp[((1 * NPV + N) * 2 + 1) * 64]);
      o[j] = mfma8_32(va, ph, o[j]);
      o[j] = mfma8_32(va, pl, o[j]);
    }
  };

  // Wait until this wave's DMAs of K(v+2) and V(v) have landed: at most the
  // tiles issued after V(v) (K(v+3), V(v+1), K(v+4), V(v+2), those that
  // exist) may still be in flight.
  auto wait_step = [&](int v) {
    const int later = (v + 3 < v_hi) + (v + 1 < v_hi) + (v + 4 < v_hi) + (v + 2 < v_hi);
    if (later == 4) wait_vmem<4 * TPW>();
    else if (later == 3) wait_vmem<3 * TPW>();
    else if (later == 2) wait_vmem<2 * TPW>();
    else if (later == 1) wait_vmem<TPW>();
    else wait_vmem<0>();
  };

  const int n_st = v_hi - v_lo;
  // First the loads that do not wait on the page table: the item's page ids
  // (for LDS), the ancestor words of this wave's columns, Q.
  int32_t pid_l = 0;
  if (wave == 0 && map.paged && t0 + lane <= t_last) pid_l = map.pt[t0 + lane];
  uint32_t anc_l[NTW];
#pragma unroll
  for (int nt = 0; nt < NTW; ++nt) {
    const Col k = col_of(qcol(nt));
    anc_l[nt] = 0xFFFFFFFFu;
    if (s == 0 && a == 0 && S.tree_mask && k.ok) anc_l[nt] = S.tree_mask[k.row];
  }
  q_load();
  if (v_hi > v_lo) {
    // Prologue DMAs, in the order the steady state expects: K(v_lo),
    // K(v_lo+1); then as "step v_lo-2" K(v_lo+2), V(v_lo), and as "step
    // v_lo-1" K(v_lo+3), V(v_lo+1).  All lie in the item's first page.
    dma_k(v_lo);
    if (n_st > 1) dma_k(v_lo + 1);
    if (n_st > 2) dma_k(v_lo + 2);
    dma_v(v_lo);
    if (n_st > 3) dma_k(v_lo + 3);
    if (n_st > 1) dma_v(v_lo + 1);
  }
  // Q operands, ancestor words and the page ids, while the first tiles load
  q_split();
#pragma unroll
  for (int j = 0; j < NPW; ++j) o[j] = v16f{};
#pragma unroll
  for (int nt = 0; nt < NTW; ++nt)
    if (s == 0 && a == 0) Anc[qcol(nt)] = anc_l[nt];
  if (wave == 0 && map.paged) Pid[lane] = pid_l;

  if (v_hi > v_lo) {
    // K(v_lo) and K(v_lo+1) landed: after them at most K(v_lo+2), V(v_lo),
    // K(v_lo+3), V(v_lo+1) remain
    {
      const int later = (n_st > 2) + 1 + (n_st > 3) + (n_st > 1);
      if (later == 4) wait_vmem<4 * TPW>();
      else if (later == 3) wait_vmem<3 * TPW>();
      else if (later == 2) wait_vmem<2 * TPW>();
      else wait_vmem<TPW>();
    }
    lds_barrier();
    // The logits of two steps are live at a time: in interval v those of
    // step v-1 (for the slow path of its check) and of step v, and S(v+1)
    // takes step v-1's registers once that check is done.  Intervals run in
    // pairs with the two buffers' roles swapped.
    v4f B0[NTW], B1[NTW];
    qk(v_lo, B0);
    lds_barrier();  // every wave is done with K(v_lo) before K(v_lo+4) reuses its stage

    // Interval v runs between barriers v-1 and v: the DMAs of K(v+4) and
    // V(v+2), the check and the P.V of step v-1, the softmax of step v and
    // S(v+1).
    auto steady = [&](int v, v4f (&X)[NTW], v4f (&Y)[NTW]) __attribute__((always_inline)) {
      // the V operand's reads go out with the flag read, under one wait
      const v8i va = pv_prep(v - 1, false);
      check(v - 1, X);
      if (v + 4 < v_hi) dma_k(v + 4);
      // the P.V products of step v-1 and the softmax of step v: one
      // branch-free block, each MFMA followed by a share of the VALU work.
      // The block runs at a raised issue priority (2% faster than none;
      // raising it for the QK products instead, or for one wave of each
      // SIMD throughout, gained less).
      __builtin_amdgcn_s_setprio(2);
      pv_body(v - 1, va);
      soft(v, Y, true);
      __builtin_amdgcn_sched_group_barrier(kDsRead, 4, 1);
#pragma unroll
      for (int i = 0; i < 2 * NPW; ++i) {
        __builtin_amdgcn_sched_group_barrier(kMfma, 1, 1);
        __builtin_amdgcn_sched_group_barrier(kValu, 10, 1);
        __builtin_amdgcn_sched_group_barrier(kDsRead, 2, 1);
      }
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_setprio(0);
      if (v + 2 < v_hi) dma_v(v + 2);
      qk(v + 1, X);
      wait_step(v);
      lds_barrier();  // publishes P(v), its flags, K(v+2), V(v)
    };

    // interval v_lo: no P.V yet
    if (v_lo + 4 < v_hi) dma_k(v_lo + 4);
    if (v_lo + 2 < v_hi) dma_v(v_lo + 2);
    soft(v_lo, B0, true);
    if (v_lo + 1 < v_hi) {
      qk(v_lo + 1, B1);
    } else {
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt) B1[nt] = B0[nt];  // the last step's logits are in B1
    }
    wait_step(v_lo);
    lds_barrier();
    // steady intervals v_lo+1 .. v_hi-2: from here, at the start of an even
    // count of them, S(v-1) is in B0 and S(v) in B1
    int v = v_lo + 1;
    if (n_st > 2 && ((n_st - 2) & 1)) {
      steady(v, B0, B1);
      ++v;
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt) {
        const v4f t = B0[nt];
        B0[nt] = B1[nt];
        B1[nt] = t;
      }
    }
    for (; v + 2 < v_hi; v += 2) {
      steady(v, B0, B1);
      steady(v + 1, B1, B0);
    }
    // interval v_hi - 1 (when it is not v_lo): check and P.V of v_hi - 2, the last softmax
    if (v_hi - 1 > v_lo) {
      check(v_hi - 2, B0);
      pv_body(v_hi - 2, pv_prep(v_hi - 2, false));
      soft(v_hi - 1, B1, true);
      wait_step(v_hi - 1);
      lds_barrier();
    }
    // the last interval: check and P.V of step v_hi - 1, past the stream's end zeroed
    check(v_hi - 1, B1);
    pv_body(v_hi - 1, pv_prep(v_hi - 1, (v_hi - 1) * BK + BK > n_keys_t));
  }

  // A rejected page id (out of the pool) anywhere in the item poisons its
  // partials: checked here, one id per lane, rather than carried through the
  // step loop.  (The tiles of such pages read page 0 instead.)
  bool bad_lane = false;
  if (map.paged && v_hi > v_lo) {
    if (t_last - t0 < 64) {
      // the item's page ids are in LDS
      if (lane <= t_last - t0) bad_lane = (uint32_t)Pid[lane] >= (uint32_t)map.n_pages;
    } else {
      for (int t = t0 + lane; t <= t_last; t += 64) bad_lane |= (uint32_t)map.pt[t] >= (uint32_t)map.n_pages;
    }
  }
  const bool bad = __any(bad_lane);

  // Row sums: each wave's partial over its keys (summed across the column's
  // four lane groups), then, for every column, the four SIMDs' sums in SIMD
  // order.
#pragma unroll
  for (int nt = 0; nt < NTW; ++nt) {
    const float l = rows4_sum(l_part[nt]);
    if (a == 0) Mx[qcol(nt) * 4 + s] = l;
  }
  lds_barrier();
  if (s == 0 && a == 0) {
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) {
      const Col k = col_of(qcol(nt));
      if (!k.ok) continue;
      const int64_t slot =
          S.slot_base + ((int64_t)k.row * A.n_q_heads + k.head) * S.n_splits + split;
      const v4f l4 = *reinterpret_cast<const v4f*>(Mx + qcol(nt) * 4);
      // p was 2^(s*cc - mc): the split's reference logit in log2 units is mc
      // (minus infinity when the column saw no key); a rejected page id
      // poisons it as a NaN
      const float mref = mc[nt] == kNoMax ? -INFINITY : mc[nt];
      A.ws_ml[2 * slot] = bad ? __builtin_nanf("") : mref;
      A.ws_ml[2 * slot + 1] = ((l4[0] + l4[1]) + l4[2]) + l4[3];
    }
  }
  // o: lane (c, grp) of n-tile j holds dims DS*s + 32mt + 8q + 4grp + r
#pragma unroll
  for (int j = 0; j < NPW; ++j) {
    const Col k = col_of(32 * (n0_w + j) + c32);
    if (!k.ok) continue;
    const int64_t slot =
        S.slot_base + ((int64_t)k.row * A.n_q_heads + k.head) * S.n_splits + split;
    float* dst = A.ws_o + slot * D + DS * s + 32 * mt_w + 4 * g32;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      *reinterpret_cast<v4f*>(dst + 8 * q) =
          v4f{o[j][4 * q], o[j][4 * q + 1], o[j][4 * q + 2], o[j][4 * q + 3]};
  }
}

template <int D>
static int launch_verify_t(const PrefillArgs& A, hipStream_t st) {
  dim3 grid((unsigned)(A.total_tiles * A.cache.n_kv_heads * (A.group / A.heads_per_wg)));
  hipLaunchKernelGGL((verify_kernel<D>), grid, dim3(512), 0, st, A);
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

int verify_wg_columns(int head_dim) { return 2 * 16 * verify_ntiles(head_dim); }

int launch_verify(const PrefillArgs& A, int head_dim, hipStream_t st) {
  if (head_dim == 128) return launch_verify_t<128>(A, st);
  if (head_dim == 256) return launch_verify_t<256>(A, st);
  return -7;
}

}  // namespace pa
