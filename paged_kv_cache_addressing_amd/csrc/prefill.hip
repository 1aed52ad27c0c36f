// Causal prompt-chunk prefill over a paged (or slab) prefix for gfx950.
//
// The prompt rows read the cache through the page table, with the page size
// a compile-time constant of 256 and one page lookup per page (TensorFold
// pull request #1373, prompt rows; pull request #2011, the 256-position
// prompt kernel and the commit that looks a paged item's page up once
// instead of per 16-byte chunk).  Keys past a row's limit contribute zeros
// (pull request #2011 review, "Is paged output the same as windowed
// output?").
//
// Work split.  A workgroup owns one kv head, HW of its q heads and a tile of
// query rows; its column groups own 16*NT MFMA columns each, a column being
// one (row, q head) pair (column c of the workgroup is (c / HW, c % HW)).
// At head_dim 256: 4 column groups, each a producer/consumer wave pair on
// one SIMD, of three n-tiles (prefill) or two (split mode); at 128: 4 waves
// of three n-tiles, each running both phases.  The K/V tiles in LDS serve all HW heads, and
// the other head groups of the same kv head run on the same XCD, so K/V
// also hit in L2.
//   S^T (32 keys x 16NT cols) = K Q^T    : 2 m-tiles x NT n-tiles x D/32 k-steps
//   O^T (D x 16NT cols)      += V^T P^T  : D/16 m-tiles x NT n-tiles x 1 k-step
// The key order inside a step is permuted so each lane's S^T C-rows are the
// 8 consecutive keys of its P^T operand (no shuffles between the products).
//
// Split mode (decode streams with many rows, e.g. speculative verify rows):
// the same kernel computes one split_keys-key split of a row tile covering
// the whole group (16 rows x 6 heads = 96 columns), so each split's K/V is
// read from HBM once for all its columns, and writes the split's (m, l, o)
// partial for the log-sum-exp merge (TensorFold issue #1344, "Mechanism").
// Rows may carry an ancestor table (draft trees; pull request #1355,
// follow-up checks, "Indexing"): then, of the rows' own keys, a row sees
// only those its word marks.
//
// Pipeline.  K and V steps (32 keys) rotate through three K and four V LDS
// slots, in "fragment order" (the 1 KiB an MFMA operand needs is contiguous,
// lane l's 16 bytes at l*16, so ds_read_b128 is conflict-free).  bf16 arrives
// by buffer_load_dwordx4 ... lds straight into LDS, two steps ahead; fp8 codes
// arrive the same way into a staging ring three steps ahead and are
// converted to bf16 fragment order once, one step ahead.  In step v the
// S product S(v+1) = K(v+1) Q^T runs on the matrix cores while the VALU does
// the softmax of S(v); O += V(v) P(v) follows in the same wave, or (wave
// pairs) in the consumer wave one step later.  With pairs, bf16 K/V DMAs are
// issued and awaited by the consumer waves only; fp8 in split mode, when the
// last column group holds no column, is loaded and converted by that idle
// pair alone.
//
// Softmax.  Logits stay raw until exp2(fma(s, c, -m c)).  A row's running max
// moves only when the new maximum exceeds it by more than 2^8 in probability
// (p <= 256 otherwise), so the O accumulators are almost never rescaled.  The
// rule is per row and a rescale by exactly 1 is the identity, so no row's
// bytes depend on its neighbours.
//
// Row independence: a row's arithmetic depends only on its own position and
// the keys; key steps run from key 0 in a fixed order, and a step wholly
// masked for a row leaves its state bit-identical (max unchanged, alpha = 1,
// p = 0 against finite or zeroed values).  So any slicing of a stream's rows
// across calls gives the same bytes as one call.
#include <type_traits>

#include "pa_device.hpp"
#include "pa_internal.hpp"

namespace pa {

template <int KV, int D, bool SPLIT>
__global__ __launch_bounds__(64 * prefill_waves(D), 1) void prefill_kernel(const PrefillArgs A) {
  // A workgroup owns one kv head g, HW = heads_per_wg of its q heads (head
  // group hg) and a tile of rpt rows: its 4*16*NT columns, numbered
  // c = 16*NT*wave + 16*nt + n, are the (row, head) pairs (c / HW, c % HW).
  constexpr int ESZ = KV ? 1 : 2;
  constexpr int BK = 32;                // keys per step
  constexpr int MT = 2;                 // S^T m-tiles per step
  constexpr int KS = D / 32;            // QK k-steps
  constexpr int MD = D / 16;            // O^T m-tiles
  constexpr bool PAIR = prefill_paired(KV, D);  // producer/consumer wave pairs
  constexpr int NT = prefill_ntiles(KV, D, SPLIT);  // 16-column n-tiles per column group
  constexpr int NG = prefill_groups(KV, D);  // column groups per workgroup
  constexpr int NW = prefill_waves(D);   // waves per workgroup
  constexpr int NTH = 64 * NW;          // threads per workgroup
  constexpr int KF = MT * KS;           // K fragments (1 KiB) per step
  constexpr int VF = MD;                // V fragments per step
  // bf16 with wave pairs: only the consumer waves (P.V, no softmax) issue
  // and await the K/V DMAs, so the producers' S/softmax phase carries none.
  constexpr bool CLOAD = KV == 0 && PAIR;
  constexpr int NLB = CLOAD ? NG : NW;  // bf16 loader waves
  constexpr int KPW = KF / NLB;         // DMA fragments per loader wave per step
  constexpr int VPW = VF / NLB;
  // K and V slot rings (see the step schedule): bf16 DMAs K three and V two
  // steps ahead; fp8 converts K(v+2) and V(v+1) into their slots in step v.
  constexpr int NSLOT = KV ? 2 : 3;     // K slots
  constexpr int NVSLOT = KV ? 3 : 4;    // V slots
  constexpr int KSLOT = KF * 64;        // 16-byte entries per slot
  constexpr int VSLOT = VF * 64;
  // fp8: raw codes land in a staging ring (16-byte entries per step) and are
  // converted to bf16 fragment order from there.
  constexpr int KST = KF * 64 / 2;
  constexpr int VST = VF * 64 / 2;
  constexpr int NSTG = 3;
  static_assert(KST % (64 * NW) == 0 && VST % (64 * NW) == 0, "fp8 entries per loader wave");
  static_assert(kPage % BK == 0, "a step never straddles two pages");

  // Paired waves hand P (bf16, fragment order) and the rescale factors from
  // producer to consumer through a two-slot ring per column group.
  constexpr int PSLOT = NG * NT * 64;   // 16-byte entries per P slot
  constexpr int ASLOT = NG * NT * 16;   // floats per rescale-factor slot
  __shared__ v4u lds[NSLOT * KSLOT + NVSLOT * VSLOT + (KV ? NSTG * (KST + VST) : 0) +
                     (PAIR ? 2 * PSLOT + 2 * ASLOT / 4 : 0)];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: SGPR arithmetic
  const int n = lane & 15;
  const int a = lane >> 4;
  const int G = A.group;
  const int HW = A.heads_per_wg;
  const int rpt = A.rows_per_tile;
  constexpr bool split_mode = SPLIT;  // the host launches this instance iff split_keys > 0

  // Logical work item: (kv head, head group) major, then items (prefill:
  // row tiles longest first; split mode: split_item).  With the remap, the
  // blocks one XCD runs (blockIdx % 8 picks the XCD) come from one head
  // group, whose K/V then hit in that XCD's L2.  When a head group's tiles
  // fill m whole XCDs, its tiles, longest first, are dealt to them in
  // snake order (0 1 .. m-1, m-1 .. 1 0, ...), so the m XCDs get equal
  // sums of work rather than the longest tiles going to the first of them.
  const int nb = gridDim.x;
  int L = (int)blockIdx.x;
  if (A.xcd_remap) {
    const int x = (int)(blockIdx.x % 8), sl = (int)(blockIdx.x / 8), C = nb / 8;
    if (!split_mode && A.total_tiles % C == 0) {
      const int m = A.total_tiles / C;
      const int off = x % m;
      L = (x / m) * A.total_tiles + sl * m + ((sl & 1) ? m - 1 - off : off);
    } else {
      L = x * C + sl;
    }
  }
  int hgrp, si, tile, split;  // hgrp = kv head * (G / HW) + head group
  if (split_mode) {
    split_item(A, L, nb, hgrp, si, tile, split);
  } else {
    hgrp = L / A.total_tiles;
    const int it = A.total_tiles - 1 - L % A.total_tiles;
    si = find_stream<0>(A.s, A.n_streams, it);
    tile = it - A.s[si].block_begin;
    split = 0;
  }
  const int g = hgrp / (G / HW);
  const int h0 = g * G + (hgrp % (G / HW)) * HW;
  const StreamArg& S = A.s[si];
  const int row0 = tile * rpt;
  const int rows_here = min(rpt, S.n_rows - row0);
  const int pos_first = S.first_pos + row0;
  const int pos_last = pos_first + rows_here - 1;
  const int n_keys_t = pos_last + 1;       // keys the tile's last row sees
  // Steps [v_lo, v_hi) of 32 keys: all keys the tile sees, or one split of them.
  const int k_lo = split * A.split_keys;
  const int k_end = split_mode ? min(k_lo + A.split_keys, n_keys_t) : n_keys_t;
  const int v_lo = k_lo / BK;
  const int v_hi = k_end > k_lo ? (k_end + BK - 1) / BK : v_lo;
  // Column group of this wave; with pairs, waves g and g + NG share group g
  // (and a SIMD): g is the producer, g + NG the consumer.
  const int cg = PAIR ? wave % NG : wave;
  const bool producer = !PAIR || wave < NG;
  const bool wave_active = cg * 16 * NT < rows_here * HW;
  // first key some row of the tile may not see: past the first row's own
  // position, or (ancestor table) the stream's first row key
  const int mask_from = S.tree_mask ? S.first_pos : pos_first + 1;

  // Column nt of this wave: its q head, its row (absolute in the stream),
  // whether the row is in the tile, and the last key it sees.  Recomputed
  // where needed from an opaque copy of the lane index, so none of it stays
  // in registers through the step loop.
  struct Col {
    int row, head, pos;
    bool ok;
  };
  auto col = [&](int nt) -> Col {
    int ln = n;
    asm("" : "+v"(ln));
    const int c = 16 * NT * cg + 16 * nt + ln;
    const int rl = c / HW;
    Col k;
    k.head = h0 + (c - rl * HW);
    k.row = row0 + rl;
    k.ok = rl < rows_here;
    k.pos = k.ok ? S.first_pos + k.row : pos_last;
    return k;
  };
  // Q^T fragments of this wave's columns (loaded by the waves that run the S
  // product, inside their own copy of the step loop).
  v8bf qb[NT][KS];
  auto load_q = [&]() {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const Col k = col(nt);
      const uint8_t* qp = reinterpret_cast<const uint8_t*>(A.q) +
                          ((int64_t)(S.row_offset + (k.ok ? k.row : row0)) * A.n_q_heads +
                           (k.ok ? k.head : h0)) * D * 2;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int d0 = KV ? 64 * (ks >> 1) + 16 * a + 8 * (ks & 1) : 32 * ks + 8 * a;
        v4u x = load16(qp + d0 * 2);
        if (!k.ok) x = v4u{0, 0, 0, 0};
        qb[nt][ks] = as_bf(x);
      }
    }
  };

  v4u* const Kbase = lds;
  v4u* const Vbase = lds + NSLOT * KSLOT;
  // The same slots as LDS-address-space pointers: 32-bit LDS addresses, so a
  // fragment's constant offset folds into the ds_read immediate.
  typedef __attribute__((address_space(3))) v4u lds_v4u;
  lds_v4u* const Kb3 = (lds_v4u*)Kbase;
  lds_v4u* const Vb3 = (lds_v4u*)Vbase;
  // Per-lane base of a slot, kept opaque so the compiler cannot reassociate
  // the constant fragment offsets away from the ds_read immediate field.
  auto lane_base = [&](lds_v4u* slot0, int slot) -> const lds_v4u* {
    uint32_t addr = (uint32_t)(uintptr_t)(slot0 + slot + lane);
    asm("" : "+v"(addr));
    return (const lds_v4u*)(uintptr_t)addr;
  };
  // The K loader runs ahead of the V loader; each keeps its own page, so
  // every page is looked up once per loader.
  PageTile TK{}, TV{};
  int pk = -1, pvp = -1;
  bool bad = false;
  auto page_k = [&](int v) -> const PageTile& {
    if ((v >> 3) != pk) {
      pk = v >> 3;
      TK = page_tile<D, ESZ>(S, A.cache, pk, g);
      bad |= !TK.ok;
    }
    return TK;
  };
  auto page_v = [&](int v) -> const PageTile& {
    if ((v >> 3) != pvp) {
      pvp = v >> 3;
      TV = page_tile<D, ESZ>(S, A.cache, pvp, g);
      bad |= !TV.ok;
    }
    return TV;
  };
  // S^T row m of m-tile mt holds key 8*(m/4) + 4*mt + m%4 of the step.
  const int krow = 8 * (n >> 2) + (n & 3);

  // bf16 loaders: loader wave lb DMAs KPW K fragments and VPW V fragments.
  const bool bl = !CLOAD || !producer;
  const int lb = CLOAD ? cg : wave;
  // Each DMA is the step's base in the page tile (o*D*2 bytes for both K
  // and V: wave-uniform, SGPRs) plus a per-lane offset that does not depend
  // on the step (loop invariant, hoisted into VGPRs).
  auto dma_k = [&](int v, int sl) {
    const PageTile& T = page_k(v);
    const auto rs = tile_rsrc(T.k, kPage * D * 2);
    const int soff = (v & 7) * BK * D * 2;
    v4u* dst = Kbase + sl * KSLOT + lb * KPW * 64;
#pragma unroll
    for (int i = 0; i < KPW; ++i) {
      const int f = lb * KPW + i, mt = f / KS, ks = f % KS;
      const int off = ((krow + 4 * mt) * D + 32 * ks + 8 * a) * 2;
      dma16(rs, off, soff, dst + i * 64);
    }
  };
  auto dma_v = [&](int v, int sl) {
    const PageTile& T = page_v(v);
    const auto rs = tile_rsrc(T.v, kPage * D * 2);
    const int soff = (v & 7) * BK * D * 2;
    v4u* dst = Vbase + sl * VSLOT + lb * VPW * 64;
#pragma unroll
    for (int i = 0; i < VPW; ++i) {
      const int off = v_off<D, ESZ>(8 * a, 16 * (lb * VPW + i) + n) * 2;
      dma16(rs, off, soff, dst + i * 64);
    }
  };
  // bf16 tail: values at or past n_keys_t in a landed V step become zeros.
  auto zero_tail_bf16 = [&](int v, int sl) {
    v4u* Ls = Vbase + sl * VSLOT;
#pragma unroll
    for (int i = 0; i < VSLOT / NTH; ++i) {
      const int q = i * NTH + tid, lp = q & 63;
      Ls[q] = keep_first_h(Ls[q], n_keys_t - (v * BK + 8 * (lp >> 4)));
    }
  };

  // fp8 loaders.  Raw codes are DMAed into the staging ring (K four steps
  // and V three steps before their use), each 16-byte entry by the wave that
  // converts it; the conversion to bf16 fragment order then runs one step
  // ahead of use (K two steps).  Every E4M3FN value is a bf16 value, so the
  // conversion is exact.
  //
  // Loader waves.  Normally all NW waves share the staging entries.  In
  // split mode, when the last column group holds no column (96 verify
  // columns in 128), its two waves are the only loaders: they issue every DMA, wait for
  // it and convert it, and the column-holding waves only compute and pass
  // the barriers.  Loader wave li of NL takes K entry groups li, li + NL, ...
  // and V entries (li * 64 + lane) + 64 NL i.
  const bool ded = SPLIT && KV == 1 && PAIR && (NG - 1) * 16 * NT >= rows_here * HW;
  const bool loader = !ded || cg == NG - 1;
  const int li = ded ? (producer ? 0 : 1) : wave;
  typedef std::integral_constant<int, NW> AllLoad;
  typedef std::integral_constant<int, 2> PairLoad;
  v4u* const Sbase = lds + NSLOT * KSLOT + NVSLOT * VSLOT;
  auto dma8_k = [&](int v, int sl, auto nl) __attribute__((always_inline)) {
    constexpr int NL = decltype(nl)::value;
    const PageTile& T = page_k(v);
    const auto rs = tile_rsrc(T.k, kPage * D);
    const int soff = (v & 7) * BK * D;
    v4u* dst = Sbase + sl * (KST + VST);
#pragma unroll
    for (int i = 0; i < KST / 64 / NL; ++i) {
      // entry fp*64 + lane: 16 dims (two QK k-steps) of one S^T row
      const int fp = NL * i + li, mt = fp / (KS / 2), kq = fp % (KS / 2);
      const int off = (krow + 4 * mt) * D + 64 * kq + 16 * a;
      dma16(rs, off, soff, dst + fp * 64);
    }
  };
  auto dma8_v = [&](int v, int sl, auto nl) __attribute__((always_inline)) {
    constexpr int NL = decltype(nl)::value;
    const PageTile& T = page_v(v);
    const int o = (v & 7) * BK;
    const auto rs = tile_rsrc(T.v, kPage * D);
    v4u* dst = Sbase + sl * (KST + VST) + KST;
#pragma unroll
    for (int i = 0; i < VST / 64 / NL; ++i) {
      // entry q: 16 keys (half h of the step) of dim 16*md + dl
      const int q = i * 64 * NL + li * 64 + lane, md = q >> 5, dl = q & 15, h = (q >> 4) & 1;
      const int off = v_off<D, ESZ>(o + 16 * h, 16 * md + dl);
      dma16(rs, off, 0, dst + (q >> 6) * 64);
    }
  };
  auto convert_fp8 = [&](int vk, int stk, int slk, int vv, int stv, int slv, auto may_tail,
                         auto nl) __attribute__((always_inline)) {
    constexpr int NL = decltype(nl)::value;
    if (vk >= 0) {
      const v4u* St = Sbase + stk * (KST + VST);
      v4u* Ls = Kbase + slk * KSLOT;
#pragma unroll
      for (int i = 0; i < KST / 64 / NL; ++i) {
        const int fp = NL * i + li, mt = fp / (KS / 2), kq = fp % (KS / 2);
        const int f0 = mt * KS + 2 * kq;
        const v4u x = St[fp * 64 + lane];
        Ls[f0 * 64 + lane] = __builtin_bit_cast(v4u, fp8x8_to_bf16(x[0], x[1]));
        Ls[(f0 + 1) * 64 + lane] = __builtin_bit_cast(v4u, fp8x8_to_bf16(x[2], x[3]));
      }
    }
    if (vv >= 0) {
      const v4u* St = Sbase + stv * (KST + VST) + KST;
      v4u* Ls = Vbase + slv * VSLOT;
      const bool tail = decltype(may_tail)::value && vv * BK + BK > n_keys_t;
#pragma unroll
      for (int i = 0; i < VST / 64 / NL; ++i) {
        const int q = i * 64 * NL + li * 64 + lane, md = q >> 5, dl = q & 15, h = (q >> 4) & 1;
        v4u x = St[q];
        if (tail) x = keep_first_b(x, n_keys_t - (vv * BK + 16 * h));
        Ls[md * 64 + 32 * h + dl] = __builtin_bit_cast(v4u, fp8x8_to_bf16(x[0], x[1]));
        Ls[md * 64 + 32 * h + 16 + dl] = __builtin_bit_cast(v4u, fp8x8_to_bf16(x[2], x[3]));
      }
    }
  };

  v4f o[MD][NT];
#pragma unroll
  for (int md = 0; md < MD; ++md)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) o[md][nt] = v4f{0.f, 0.f, 0.f, 0.f};
  float m_run[NT], l_run[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    m_run[nt] = -INFINITY;
    l_run[nt] = 0.f;
  }
  const float c = A.scale_log2;
  const float thr = 8.f / c;  // move the max only past p = 2^8

  auto mask = [&](int v, v4f (&Sx)[MT][NT]) {
    const int kabs0 = v * BK + 8 * a;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const Col k = col(nt);
      // ancestor word of the column's row (all ones: causal chain)
      const uint32_t anc = (S.tree_mask && k.ok) ? S.tree_mask[k.row] : 0xFFFFFFFFu;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          // branch-free: a select per logit (nested conditions here were
          // compiled into control flow that dropped the ancestor test)
          const int kabs = kabs0 + 4 * mt + i, rel = kabs - S.first_pos;
          const bool anc_ok = (rel < 0) | (((anc >> (rel & 31)) & 1u) != 0u);
          const bool vis = (kabs <= k.pos) & anc_ok;
          Sx[mt][nt][i] = vis ? Sx[mt][nt][i] : -INFINITY;
        }
    }
  };

  // S(v+1) = K(v+1) Q^T on the matrix cores with the softmax of S(v) on the
  // VALU, in a fixed interleaved order.  With one wave per SIMD nothing else
  // hides latency, so the order is pinned with sched_barrier: the K fragment
  // reads run RA fragments ahead of their MFMAs (a ring of RA+1 registers),
  // and the softmax is cut into 5*NT chunks spread between the MFMAs, where
  // the VALU work issues while the matrix cores are busy.
  //   chunk k <  NT      : row max over the lane's 8 logits of n-tile k
  //   chunk k < 2NT      : the max over the column's four lane rows, the new
  //                        running max (moved only past p = 2^8), alpha
  //   chunk k < 2NT+MT*NT: p = exp2(s*c - m*c) for 4 logits, partial sums
  //   else               : l update and the bf16 P^T operand
  constexpr int RA = 4;                  // LDS reads in flight ahead of use
  constexpr int NCH = 5 * NT;            // softmax chunks
  auto qk_softmax = [&](int kslot, v4f (&Sn)[MT][NT], v4f (&Sc)[MT][NT], v8bf (&P)[NT],
                        float (&alpha)[NT]) {
    const lds_v4u* Lk = lane_base(Kb3, kslot);  // fragment f at Lk[f * 64]
    float mx[NT], mc[NT], ps[NT];
    auto chunk = [&](int k) {
      if (k < NT) {
        const int nt = k;
        mx[nt] = fmaxf(fmaxf(fmaxf(Sc[0][nt][0], Sc[0][nt][1]), fmaxf(Sc[0][nt][2], Sc[0][nt][3])),
                       fmaxf(fmaxf(Sc[1][nt][0], Sc[1][nt][1]), fmaxf(Sc[1][nt][2], Sc[1][nt][3])));
      } else if (k < 2 * NT) {
        const int nt = k - NT;
        const float m = rows4_max(mx[nt]);
        float mu = m_run[nt];
        if (m > mu + thr) mu = m;
        alpha[nt] = mu == m_run[nt] ? 1.f : __builtin_amdgcn_exp2f((m_run[nt] - mu) * c);
        m_run[nt] = mu;
        mc[nt] = mu == -INFINITY ? 0.f : mu * c;
        ps[nt] = 0.f;
      } else if (k < 2 * NT + MT * NT) {
        const int nt = (k - 2 * NT) / MT, mt = (k - 2 * NT) % MT;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(Sc[mt][nt][i], c, -mc[nt]));
          Sc[mt][nt][i] = p;
          ps[nt] += p;
        }
      } else {
        const int nt = k - 2 * NT - MT * NT;
        l_run[nt] = l_run[nt] * alpha[nt] + ps[nt];
        v4u x;
        x[0] = pack_bf2(Sc[0][nt][0], Sc[0][nt][1]);
        x[1] = pack_bf2(Sc[0][nt][2], Sc[0][nt][3]);
        x[2] = pack_bf2(Sc[1][nt][0], Sc[1][nt][1]);
        x[3] = pack_bf2(Sc[1][nt][2], Sc[1][nt][3]);
        // keep P here: otherwise the exponentials sink past the rescale
        // branch, next to the P.V products that consume them
        asm volatile("" : "+v"(x));
        P[nt] = as_bf(x);
      }
    };
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) Sn[mt][nt] = v4f{0.f, 0.f, 0.f, 0.f};
    // visit order j = ks * MT + mt reads fragment mt * KS + ks
    v4u fb[RA + 1];
#pragma unroll
    for (int j = 0; j < RA; ++j) fb[j] = Lk[((j % MT) * KS + j / MT) * 64];
#pragma unroll
    for (int j = 0; j < KF; ++j) {
      if (j + RA < KF) {
        const int f = j + RA;
        fb[f % (RA + 1)] = Lk[((f % MT) * KS + f / MT) * 64];
      }
      const int ks = j / MT, mt = j % MT;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        Sn[mt][nt] = mfma16(as_bf(fb[j % (RA + 1)]), qb[nt][ks], Sn[mt][nt]);
      // softmax chunks placed after this fragment: k with slot(k) == j
#pragma unroll
      for (int k = 0; k < NCH; ++k)
        if ((k + 1) * KF / (NCH + 1) == j) chunk(k);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // O^T += V(v)^T P^T: 16-dim V fragments read RA ahead of their MFMAs.
  auto pv = [&](int vslot, v8bf (&P)[NT]) {
    const lds_v4u* Lv = lane_base(Vb3, vslot);  // fragment md at Lv[md * 64]
    v4u fb[RA + 1];
#pragma unroll
    for (int j = 0; j < RA; ++j) fb[j] = Lv[j * 64];
#pragma unroll
    for (int md = 0; md < VF; ++md) {
      if (md + RA < VF) fb[(md + RA) % (RA + 1)] = Lv[(md + RA) * 64];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        o[md][nt] = mfma16(as_bf(fb[md % (RA + 1)]), P[nt], o[md][nt]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Prologue helper: S(v_lo) alone (no softmax to overlap yet).
  auto qk = [&](int kslot, v4f (&Sx)[MT][NT]) {
    const lds_v4u* Lk = lane_base(Kb3, kslot);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) Sx[mt][nt] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int f = 0; f < KF; ++f) {
      const int mt = f / KS, ks = f % KS;
      const v4u kf = Lk[f * 64];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) Sx[mt][nt] = mfma16(as_bf(kf), qb[nt][ks], Sx[mt][nt]);
    }
  };

  // One step: issue the loads two (bf16) or one (fp8) steps ahead; S(v+1)
  // on the matrix cores alongside softmax(v) on the VALU; O += V(v) P(v);
  // and the hand-off: wait for the next steps' tiles, then a barrier that
  // publishes them and releases the slots read before it.
  // FAST is the steady state (every prefetch in range, no causal mask, no
  // key-range tail), where the step runs without any of those checks.  The
  // fp8 staging entries (and bf16 K slots) rotate with the step through three
  // ring positions, (v - v_lo) % 3, passed in as `ph` (a compile-time
  // constant in the unrolled steady state); the other rings use their own
  // period.
  //
  // Paired waves (head_dim 256).  Each column group of 32 columns has
  // a producer wave (S = K Q^T and the softmax; it holds Q, S and the running
  // max and sum) and a consumer wave on the same SIMD (O += V P^T; it holds
  // O).  In step v the producer computes P(v) and hands it over through LDS;
  // the consumer applies it in step v+1.  Each K and V fragment read from
  // LDS then feeds two MFMAs (32 columns) instead of one, which halves the
  // fragment reads per product, and the two register sets (Q and S, or O)
  // fit two waves per SIMD.
  //
  // The consumer reads V(v-1) after barrier v-1, in step v.  With bf16,
  // V(v+2) is DMAed in step v, so V has four slots (V(v-1) .. V(v+2)); K has
  // three (K(v+1) is read while K(v+2), K(v+3) land).  With fp8, step v
  // converts V(v+1) and K(v+2) from staging, so V needs three slots and K
  // two.  Every wave passes one barrier per step, in the same order.
  static_assert(NSTG == 3 && NSLOT == (KV ? 2 : 3) && NVSLOT == (KV ? 3 : 4), "ring periods");
  auto kslot = [&](int u) { return (u - v_lo) % NSLOT; };
  auto vslot = [&](int u) { return (u - v_lo) % NVSLOT; };
  // DMAs of step v; returns how many bf16 tiles were issued (0, 1 = V, 2).
  auto issue = [&](int v, auto fast, auto ph) __attribute__((always_inline)) -> int {
    constexpr bool FAST = decltype(fast)::value;
    const int r0 = ph % 3, r1 = (ph + 1) % 3;  // staging of v+3, v+4
    int issued = 0;
    if (KV == 0) {
      if (FAST || v + 2 < v_hi) {
        if (bl) dma_v(v + 2, vslot(v + 2));
        issued = 1;
      }
      if (FAST || v + 3 < v_hi) {
        if (bl) dma_k(v + 3, kslot(v + 3));
        issued = 2;
      }
    } else {
      auto load = [&](auto nl) __attribute__((always_inline)) {
        constexpr int NL = decltype(nl)::value;
        constexpr int K8 = KST / 64 / NL, V8 = VST / 64 / NL;  // DMAs per lane per step
        if (FAST || v + 4 < v_hi) dma8_k(v + 4, r1, nl);
        if (FAST || v + 3 < v_hi) dma8_v(v + 3, r0, nl);
        // Then convert K(v+2) and V(v+1) (staging positions r2 and r1) into
        // their bf16 slots at the start of the step, so the conversion
        // overlaps this step's products on the SIMD's other wave; barrier v
        // publishes them.  Their codes have landed once at most the DMAs
        // issued in steps v-1 and v (K(v+3), V(v+2), K(v+4), V(v+3), those
        // that exist) remain.
        const int r2 = (ph + 2) % 3;
        const int r = v_hi - 1 - v;
        if (FAST || r >= 4) wait_vmem<2 * (K8 + V8)>();
        else if (r == 3) wait_vmem<K8 + 2 * V8>();
        else if (r == 2) wait_vmem<V8>();
        else wait_vmem<0>();
        if (FAST)
          convert_fp8(v + 2, r2, kslot(v + 2), v + 1, r1, vslot(v + 1), std::false_type{}, nl);
        else
          convert_fp8(v + 2 < v_hi ? v + 2 : -1, r2, kslot(v + 2), v + 1 < v_hi ? v + 1 : -1, r1,
                      vslot(v + 1), std::true_type{}, nl);
      };
      if (!ded) load(AllLoad{});
      else if (loader) load(PairLoad{});
    }
    return issued;
  };
  auto hand_off = [&](int v, auto fast, auto ph, int issued) {
    constexpr bool FAST = decltype(fast)::value;
    (void)ph;
    if (KV == 0) {
      if (FAST || issued == 2) wait_vmem<KPW + VPW>();
      else if (issued == 1) wait_vmem<VPW>();
      else wait_vmem<0>();
    }
    lds_barrier();
    if (!FAST && KV == 0 && v + 1 < v_hi && (v + 1) * BK + BK > n_keys_t) {
      zero_tail_bf16(v + 1, vslot(v + 1));
      lds_barrier();
    }
  };
  // O *= alpha where some column's running max moved (rarely).
  auto rescale = [&](const float (&alpha)[NT]) {
    bool moved = false;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) moved |= alpha[nt] != 1.f;
    if (__any(moved)) {
#pragma unroll
      for (int md = 0; md < MD; ++md)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) o[md][nt] *= alpha[nt];
    }
  };
  // S(v+1) and softmax(v), raising the wave's issue priority: this phase
  // (matrix products, softmax and K reads) is the longer one, so it goes
  // ahead of a P.V-only wave on the same SIMD.
  auto s_phase = [&](int v, v4f (&Sc)[MT][NT], v4f (&Sn)[MT][NT], auto fast, auto ph,
                     v8bf (&P)[NT], float (&alpha)[NT]) {
    constexpr bool FAST = decltype(fast)::value;
    if (!FAST && v * BK + BK - 1 >= mask_from) mask(v, Sc);
    __builtin_amdgcn_s_setprio(1);
    // K(v+1), or stale data past the end (unused)
    qk_softmax(kslot(v + 1) * KSLOT, Sn, Sc, P, alpha);
    __builtin_amdgcn_s_setprio(0);
  };
  // A wave that runs both phases of its columns.
  auto step = [&](int v, v4f (&Sc)[MT][NT], v4f (&Sn)[MT][NT], auto fast, auto ph) {
    const int issued = issue(v, fast, ph);
    v8bf P[NT];
    float alpha[NT];
    if (wave_active) s_phase(v, Sc, Sn, fast, ph, P, alpha);
    if (wave_active) {
      rescale(alpha);
      pv(vslot(v) * VSLOT, P);
    }
    hand_off(v, fast, ph, issued);
  };
  // Paired waves: the P ring (slot (v - v_lo) & 1; 16 bytes per lane per
  // n-tile) and the rescale factors (one per column).
  v4u* const Pbase = lds + NSLOT * KSLOT + NVSLOT * VSLOT + (KV ? NSTG * (KST + VST) : 0);
  float* const Abase = reinterpret_cast<float*>(Pbase + 2 * PSLOT);
  auto pstep = [&](int v, v4f (&Sc)[MT][NT], v4f (&Sn)[MT][NT], auto fast, auto ph) {
    const int issued = issue(v, fast, ph);
    if (wave_active) {
      v8bf P[NT];
      float alpha[NT];
      s_phase(v, Sc, Sn, fast, ph, P, alpha);
      const int sl = (v - v_lo) & 1;
      v4u* pd = Pbase + sl * PSLOT + cg * NT * 64 + lane;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) pd[nt * 64] = __builtin_bit_cast(v4u, P[nt]);
      if (a == 0) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) Abase[sl * ASLOT + (cg * NT + nt) * 16 + n] = alpha[nt];
      }
    }
    hand_off(v, fast, ph, issued);
  };
  // O += V(u) P(u)^T with P(u) from the ring (published by barrier u).
  auto consume = [&](int u) {
    const int sl = (u - v_lo) & 1;
    const v4u* ps = Pbase + sl * PSLOT + cg * NT * 64 + lane;
    v8bf P[NT];
    float alpha[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      P[nt] = as_bf(ps[nt * 64]);
      alpha[nt] = Abase[sl * ASLOT + (cg * NT + nt) * 16 + n];
    }
    rescale(alpha);
    pv(vslot(u) * VSLOT, P);
  };
  auto cstep = [&](int v, auto fast, auto ph) {
    const int issued = issue(v, fast, ph);
    if (wave_active && v > v_lo) consume(v - 1);
    hand_off(v, fast, ph, issued);
  };

  // Output of column n-tile nt with row sum l and running max m*c (log2
  // units).
  auto write_out = [&](int nt, float l, float mc) {
    const Col k = col(nt);
    if (!k.ok) return;
    if (split_mode) {
      // Partial of (row, head, split): p was exp2(s*c - m_run*c), so the
      // split's m in log2 units is exactly m_run*c; o stays in stored-V units.
      const int64_t slot =
          S.slot_base + ((int64_t)k.row * A.n_q_heads + k.head) * S.n_splits + split;
      // A rejected page id poisons m as a NaN bit pattern (this file is built
      // without NaN semantics, so no floating-point NaN is ever formed here).
      if (a == 0) {
        const uint32_t mb = bad ? 0x7FC00000u : __builtin_bit_cast(uint32_t, mc);
        reinterpret_cast<uint32_t*>(A.ws_ml)[2 * slot] = mb;
        A.ws_ml[2 * slot + 1] = l;
      }
      float* dst = A.ws_o + slot * D + 4 * a;
#pragma unroll
      for (int md = 0; md < MD; ++md) *reinterpret_cast<v4f*>(dst + 16 * md) = o[md][nt];
      return;
    }
    const float f = A.v_scale / l;
    uint16_t* dst =
        A.out + ((int64_t)(S.row_offset + k.row) * A.n_q_heads + k.head) * D + 4 * a;
#pragma unroll
    for (int md = 0; md < MD; ++md) {
      const v4f x = o[md][nt] * f;
      v2u w;
      w[0] = pack_bf2(x[0], x[1]);
      w[1] = pack_bf2(x[2], x[3]);
      if (bad) w = v2u{0x7FC07FC0u, 0x7FC07FC0u};  // bf16 NaN bits for a rejected page id
      *reinterpret_cast<v2u*>(dst + 16 * md) = w;
    }
  };

  // The rest of the work item for one role: 0 = producer of a pair,
  // 1 = consumer of a pair, 2 = a wave that runs both phases.  Each role is
  // its own inlined copy with no path joining another role's, so the
  // registers a role does not touch (Q and S for a consumer, O for a
  // producer) are free in its copy.
  auto run = [&](auto role) {
    constexpr int R = decltype(role)::value;
    if constexpr (R != 1) load_q();
    // Prologue: K(v_lo), V(v_lo), K(v_lo+1) resident as bf16 (bf16 also has
    // K(v_lo+2), V(v_lo+1) in flight; fp8 has the codes of V(v_lo+1..v_lo+2)
    // and K(v_lo+2..v_lo+3) in flight); S(v_lo) computed; then the slot of
    // K(v_lo) may be reused.  A work item with no keys skips to its output.
    if (v_hi > v_lo) {
      const int n_st = v_hi - v_lo;
      v4f S0[MT][NT], S1[MT][NT];
      if (KV == 0) {
        if (bl) {
          dma_k(v_lo, 0);
          dma_v(v_lo, 0);
          if (n_st > 1) dma_k(v_lo + 1, 1);
          if (n_st > 1) dma_v(v_lo + 1, 1);
          if (n_st > 2) dma_k(v_lo + 2, 2);
        }
        if (n_st > 2) wait_vmem<KPW + VPW>();
        else if (n_st > 1) wait_vmem<VPW>();
        else wait_vmem<0>();
      } else {
        auto prologue = [&](auto nl) __attribute__((always_inline)) {
          dma8_k(v_lo, 0, nl);
          dma8_v(v_lo, 0, nl);
          if (n_st > 1) dma8_k(v_lo + 1, 1, nl);
          wait_vmem<0>();
          convert_fp8(v_lo, 0, 0, v_lo, 0, 0, std::true_type{}, nl);
          if (n_st > 1) convert_fp8(v_lo + 1, 1, 1, -1, 0, 0, std::true_type{}, nl);
          // the staging reads above finish before K(v_lo+3) reuses K(v_lo)'s entries
          asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
          if (n_st > 1) dma8_v(v_lo + 1, 1, nl);
          if (n_st > 2) dma8_k(v_lo + 2, 2, nl);
          if (n_st > 2) dma8_v(v_lo + 2, 2, nl);
          if (n_st > 3) dma8_k(v_lo + 3, 0, nl);
        };
        if (!ded) prologue(AllLoad{});
        else if (loader) prologue(PairLoad{});
      }
      __syncthreads();
      if (KV == 0 && v_lo * BK + BK > n_keys_t) {
        zero_tail_bf16(v_lo, 0);
        __syncthreads();
      }
      if (R != 1 && wave_active) qk(0, S0);
      __syncthreads();

      // Steps [v_lo, v_fast) are steady state: v+3 (bf16) or v+4 (fp8) is
      // still in range, no key of the step is maskable (before mask_from),
      // and the next V step holds no key at or past n_keys_t.
      const int v_fast = max(v_lo, min(min(v_hi - (KV ? 4 : 3), mask_from / BK),
                                       n_keys_t / BK - 1));
      // The steady state runs three steps per iteration, one per ring
      // position, so every slot address is a constant; S(v+1) alternates
      // between S0 and S1.
      auto copy_s = [&](v4f (&dst)[MT][NT], v4f (&src)[MT][NT]) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) dst[mt][nt] = src[mt][nt];
      };
      typedef std::integral_constant<int, 0> P0;
      typedef std::integral_constant<int, 1> P1;
      typedef std::integral_constant<int, 2> P2;
      int v = v_lo;
      if constexpr (R == 0) {
        for (; v + 3 <= v_fast; v += 3) {
          pstep(v, S0, S1, std::true_type{}, P0{});
          pstep(v + 1, S1, S0, std::true_type{}, P1{});
          pstep(v + 2, S0, S1, std::true_type{}, P2{});
          copy_s(S0, S1);
        }
        for (; v < v_hi; ++v) {
          pstep(v, S0, S1, std::false_type{}, (v - v_lo) % 3);
          copy_s(S0, S1);
        }
      } else if constexpr (R == 1) {
        for (; v + 3 <= v_fast; v += 3) {
          cstep(v, std::true_type{}, P0{});
          cstep(v + 1, std::true_type{}, P1{});
          cstep(v + 2, std::true_type{}, P2{});
        }
        for (; v < v_hi; ++v) cstep(v, std::false_type{}, (v - v_lo) % 3);
        // P(v_hi - 1), published by the last step's barrier
        if (wave_active) consume(v_hi - 1);
      } else {
        for (; v + 3 <= v_fast; v += 3) {
          step(v, S0, S1, std::true_type{}, P0{});
          step(v + 1, S1, S0, std::true_type{}, P1{});
          step(v + 2, S0, S1, std::true_type{}, P2{});
          copy_s(S0, S1);
        }
        for (; v < v_hi; ++v) {
          step(v, S0, S1, std::false_type{}, (v - v_lo) % 3);
          copy_s(S0, S1);
        }
      }
    }

    if constexpr (R == 0) {
      // The producer hands its row sums and running maxima to the consumer
      // through LDS (the K slots, free once the last step's barrier passed).
      float* X = reinterpret_cast<float*>(lds);
      if (wave_active) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const float l = rows4_sum(l_run[nt]);
          if (a == 0) {
            X[(cg * NT + nt) * 32 + n] = l;
            X[(cg * NT + nt) * 32 + 16 + n] = m_run[nt] * c;
          }
        }
      }
      // With loader waves only they looked pages up: the producer of the
      // loader pair passes on whether a page id was rejected.
      if (ded && cg == NG - 1 && lane == 0)
        reinterpret_cast<int*>(lds)[NG * NT * 32] = bad ? 1 : 0;
      __syncthreads();
    } else if constexpr (R == 1) {
      const float* X = reinterpret_cast<const float*>(lds);
      __syncthreads();
      if (!wave_active) return;
      if (ded) bad |= reinterpret_cast<const int*>(lds)[NG * NT * 32] != 0;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        write_out(nt, X[(cg * NT + nt) * 32 + n], X[(cg * NT + nt) * 32 + 16 + n]);
    } else {
      if (!wave_active) return;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) write_out(nt, rows4_sum(l_run[nt]), m_run[nt] * c);
    }
  };
  if constexpr (PAIR) {
    if (producer) run(std::integral_constant<int, 0>{});
    else run(std::integral_constant<int, 1>{});
  } else {
    run(std::integral_constant<int, 2>{});
  }
}

template <int KV, int D, bool SPLIT>
static int launch_prefill_t(const PrefillArgs& A, hipStream_t st) {
  dim3 grid((unsigned)(A.total_tiles * A.cache.n_kv_heads * (A.group / A.heads_per_wg)));
  hipLaunchKernelGGL((prefill_kernel<KV, D, SPLIT>), grid, dim3(64 * prefill_waves(D)), 0, st, A);
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

int prefill_columns(int kv_dtype, int head_dim, bool split) {
  return 16 * prefill_ntiles(kv_dtype, head_dim, split);
}
int prefill_wg_columns(int kv_dtype, int head_dim, bool split) {
  return prefill_groups(kv_dtype, head_dim) * prefill_columns(kv_dtype, head_dim, split);
}

int launch_prefill(const PrefillArgs& A, int kv_dtype, int head_dim, hipStream_t st) {
  const bool sp = A.split_keys > 0;
  if (kv_dtype == 0 && head_dim == 128)
    return sp ? launch_prefill_t<0, 128, true>(A, st) : launch_prefill_t<0, 128, false>(A, st);
  if (kv_dtype == 0 && head_dim == 256)
    return sp ? launch_prefill_t<0, 256, true>(A, st) : launch_prefill_t<0, 256, false>(A, st);
  if (kv_dtype == 1 && head_dim == 128)
    return sp ? launch_prefill_t<1, 128, true>(A, st) : launch_prefill_t<1, 128, false>(A, st);
  if (kv_dtype == 1 && head_dim == 256)
    return sp ? launch_prefill_t<1, 256, true>(A, st) : launch_prefill_t<1, 256, false>(A, st);
  return -7;
}

}  // namespace pa
