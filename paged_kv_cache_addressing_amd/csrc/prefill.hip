// Causal prompt-chunk prefill over a paged (or slab) prefix for gfx950.
//
// The prompt rows read the cache through the page table, with the page size
// a compile-time constant of 256 and one page lookup per page (TensorFold
// pull request #1373, prompt rows; pull request #2011, hpattn_p256_kernel and
// "a paged item's page looked up once").  Keys past a row's limit land as
// zeros (pull request #2011 review, "Is paged output the same as windowed
// output?").
//
// Work split.  A workgroup (4 waves) owns one kv head, HW of its q heads and
// a tile of query rows; each wave owns 16*NT MFMA columns, a column being one
// (row, q head) pair: NT = 2 at head_dim 256 (16 rows x 2 heads for a group of
// 6), NT = 3 at 128.  The K/V tiles in LDS serve all HW heads, and the other
// head groups of the same kv head run on the same XCD, so K/V also hit in L2.
//   S^T (32 keys x 16NT cols) = K Q^T    : 2 m-tiles x NT n-tiles x D/32 k-steps
//   O^T (D x 16NT cols)      += V^T P^T  : D/16 m-tiles x NT n-tiles x 1 k-step
// The key order inside a step is permuted so each lane's S^T C-rows are the
// 8 consecutive keys of its P^T operand (no shuffles between the products).
//
// Pipeline.  K and V steps (32 keys) rotate through three LDS slots each, in
// "fragment order" (the 1 KiB an MFMA operand needs is contiguous, lane l's
// 16 bytes at l*16, so ds_read_b128 is conflict-free).  bf16 arrives by
// global_load_lds_dwordx4 straight into LDS, two steps ahead; fp8 goes
// through registers one step ahead and is converted to bf16 once.  In step v
// a wave computes S(v+1) = K(v+1) Q^T on the matrix cores while the VALU does
// the softmax of S(v), then accumulates O += V(v) P(v).
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
#include "pa_device.hpp"
#include "pa_internal.hpp"

namespace pa {

// Wait until at most N of this wave's vector-memory loads are outstanding
// (LDS-DMA loads included; they complete in issue order).
template <int N>
__device__ __forceinline__ void wait_vmem() {
  if constexpr (N == 0) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  else if constexpr (N == 2) asm volatile("s_waitcnt vmcnt(2)" ::: "memory");
  else if constexpr (N == 4) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
  else if constexpr (N == 8) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
  else static_assert(N == 0, "unsupported count");
}

// Workgroup barrier for LDS hand-off only: this wave's LDS operations are
// complete, then s_barrier.  Unlike __syncthreads() it does not wait for
// outstanding vector-memory loads, so LDS-DMA prefetches stay in flight
// across it (their completion is awaited explicitly with vmcnt).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

template <int KV, int D>
__global__ __launch_bounds__(256, 1) void prefill_kernel(const PrefillArgs A) {
  // A workgroup owns one kv head g, HW = heads_per_wg of its q heads (head
  // group hg) and a tile of 4*rpw rows; a wave owns rpw rows x HW heads.
  constexpr int ESZ = KV ? 1 : 2;
  constexpr int BK = 32;                // keys per step
  constexpr int MT = 2;                 // S^T m-tiles per step
  constexpr int KS = D / 32;            // QK k-steps
  constexpr int MD = D / 16;            // O^T m-tiles
  constexpr int NT = prefill_ntiles(D);  // 16-column n-tiles per wave
  constexpr int KF = MT * KS;           // K fragments (1 KiB) per step
  constexpr int VF = MD;                // V fragments per step
  constexpr int KPW = KF / 4;           // DMA fragments per wave per step
  constexpr int VPW = VF / 4;
  constexpr int NSLOT = 3;
  constexpr int KSLOT = KF * 64;        // 16-byte entries per slot
  constexpr int VSLOT = VF * 64;
  constexpr int KLD = KF * 64 / 2 / 256;  // fp8: 16-byte K loads per thread per step
  constexpr int VLD = VF * 64 / 256;      // fp8: 8-byte V loads per thread per step
  static_assert(kPage % BK == 0, "a step never straddles two pages");

  __shared__ v4u lds[NSLOT * (KSLOT + VSLOT)];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int n = lane & 15;
  const int a = lane >> 4;
  const int G = A.group;
  const int HW = A.heads_per_wg;
  const int rpw = A.rows_per_wave;
  const int rpt = 4 * rpw;

  // Logical work item: (kv head, head group) major, row tiles longest first.
  // With the remap, the blocks one XCD runs (blockIdx % 8 picks the XCD) form
  // one contiguous logical range, i.e. one kv head, whose K/V then hit in L2.
  const int nb = gridDim.x;
  const int L = A.xcd_remap ? (int)(blockIdx.x % 8) * (nb / 8) + (int)(blockIdx.x / 8)
                            : (int)blockIdx.x;
  const int hgrp = L / A.total_tiles;      // kv head * (G / HW) + head group
  const int g = hgrp / (G / HW);
  const int h0 = g * G + (hgrp % (G / HW)) * HW;
  const int tg = A.total_tiles - 1 - L % A.total_tiles;
  const int si = find_stream<0>(A.s, A.n_streams, tg);
  const StreamArg& S = A.s[si];
  const int row0 = (tg - S.block_begin) * rpt;
  const int rows_here = min(rpt, S.n_rows - row0);
  const int pos_first = S.first_pos + row0;
  const int pos_last = pos_first + rows_here - 1;
  const int n_keys_t = pos_last + 1;
  const int n_st = (n_keys_t + BK - 1) / BK;
  const bool wave_active = wave * rpw < rows_here;

  // Columns of this wave: lc = 16*nt + n -> (local row lc / HW, head lc % HW).
  int crow[NT], chead[NT], cpos[NT];
  bool cok[NT];
  v8bf qb[NT][KS];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int lc = 16 * nt + n;
    const int rl = lc / HW;
    chead[nt] = h0 + (lc - rl * HW);
    crow[nt] = row0 + wave * rpw + rl;
    cok[nt] = rl < rpw && crow[nt] < row0 + rows_here;
    cpos[nt] = cok[nt] ? S.first_pos + crow[nt] : pos_last;
    const uint8_t* qp = reinterpret_cast<const uint8_t*>(A.q) +
                        ((int64_t)(S.row_offset + (cok[nt] ? crow[nt] : row0)) * A.n_q_heads +
                         chead[nt]) * D * 2;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int d0 = KV ? 64 * (ks >> 1) + 16 * a + 8 * (ks & 1) : 32 * ks + 8 * a;
      v4u x = load16(qp + d0 * 2);
      if (!cok[nt]) x = v4u{0, 0, 0, 0};
      qb[nt][ks] = as_bf(x);
    }
  }

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
    asm volatile("" : "+v"(addr));
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

  // bf16 loaders: each wave DMAs KPW K fragments and VPW V fragments.
  // Each DMA is the step's base in the page tile (o*D*2 bytes for both K
  // and V: wave-uniform, SGPRs) plus a per-lane offset that does not depend
  // on the step (loop invariant, hoisted into VGPRs).
  auto dma_k = [&](int v) {
    const PageTile& T = page_k(v);
    const uint8_t* base = T.k + (int64_t)(v & 7) * BK * D * 2;
    v4u* dst = Kbase + (v % NSLOT) * KSLOT + wave * KPW * 64;
#pragma unroll
    for (int i = 0; i < KPW; ++i) {
      const int f = wave * KPW + i, mt = f / KS, ks = f % KS;
      const int off = ((krow + 4 * mt) * D + 32 * ks + 8 * a) * 2;
      __builtin_amdgcn_global_load_lds(base + off, dst + i * 64, 16, 0, 0);
    }
  };
  auto dma_v = [&](int v) {
    const PageTile& T = page_v(v);
    const uint8_t* base = T.v + (int64_t)(v & 7) * BK * D * 2;
    v4u* dst = Vbase + (v % NSLOT) * VSLOT + wave * VPW * 64;
#pragma unroll
    for (int i = 0; i < VPW; ++i) {
      const int off = v_off<D, ESZ>(8 * a, 16 * (wave * VPW + i) + n) * 2;
      __builtin_amdgcn_global_load_lds(base + off, dst + i * 64, 16, 0, 0);
    }
  };
  // bf16 tail: values at or past n_keys_t in a landed V step become zeros.
  auto zero_tail_bf16 = [&](int v) {
    v4u* Ls = Vbase + (v % NSLOT) * VSLOT;
#pragma unroll
    for (int i = 0; i < VSLOT / 256; ++i) {
      const int q = i * 256 + tid, lp = q & 63;
      Ls[q] = keep_first_h(Ls[q], n_keys_t - (v * BK + 8 * (lp >> 4)));
    }
  };

  // fp8 loaders: HBM -> registers at issue, convert + ds_write at commit.
  v4u st_k[KV ? KLD : 1];
  v2u st_v[KV ? VLD : 1];
  auto issue_fp8 = [&](int vk, int vv) {
    if (vk >= 0) {
      const PageTile& T = page_k(vk);
      const int o = (vk & 7) * BK;
#pragma unroll
      for (int i = 0; i < KLD; ++i) {
        const int q = i * 256 + tid, lp = q & 63, fp = q >> 6, m = lp & 15;
        const int mt = fp / (KS / 2), kq = fp % (KS / 2);
        st_k[i] = load16(T.k + (int64_t)(o + 8 * (m >> 2) + (m & 3) + 4 * mt) * D + 64 * kq +
                         16 * (lp >> 4));
      }
    }
    if (vv >= 0) {
      const PageTile& T = page_v(vv);
      const int o = (vv & 7) * BK;
#pragma unroll
      for (int i = 0; i < VLD; ++i) {
        const int q = i * 256 + tid, lp = q & 63, md = q >> 6;
        st_v[i] = *reinterpret_cast<const v2u*>(
            T.v + v_off<D, ESZ>(o + 8 * (lp >> 4), 16 * md + (lp & 15)));
      }
    }
  };
  auto commit_fp8 = [&](int vk, int vv) {
    if (vk >= 0) {
      v4u* Ls = Kbase + (vk % NSLOT) * KSLOT;
#pragma unroll
      for (int i = 0; i < KLD; ++i) {
        const int q = i * 256 + tid, lp = q & 63, fp = q >> 6;
        const int mt = fp / (KS / 2), kq = fp % (KS / 2);
        const int f0 = mt * KS + 2 * kq;
        Ls[f0 * 64 + lp] = __builtin_bit_cast(v4u, fp8x8_to_bf16(st_k[i][0], st_k[i][1]));
        Ls[(f0 + 1) * 64 + lp] = __builtin_bit_cast(v4u, fp8x8_to_bf16(st_k[i][2], st_k[i][3]));
      }
    }
    if (vv >= 0) {
      v4u* Ls = Vbase + (vv % NSLOT) * VSLOT;
      const bool tail = vv * BK + BK > n_keys_t;
#pragma unroll
      for (int i = 0; i < VLD; ++i) {
        const int q = i * 256 + tid, lp = q & 63;
        v4u x = v4u{st_v[i][0], st_v[i][1], 0u, 0u};
        if (tail) x = keep_first_b(x, n_keys_t - (vv * BK + 8 * (lp >> 4)));
        Ls[q] = __builtin_bit_cast(v4u, fp8x8_to_bf16(x[0], x[1]));
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

  // The LDS reads of a product are issued in batches of FB fragments, the
  // next batch in flight while the current one feeds the matrix cores, so
  // LDS latency overlaps MFMA work instead of stalling before every MFMA.
  constexpr int FB = 4;
  auto qk = [&](int kslot, v4f (&Sx)[MT][NT]) {
    const lds_v4u* Lk = lane_base(Kb3, kslot);  // fragment f at Lk[f * 64]
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) Sx[mt][nt] = v4f{0.f, 0.f, 0.f, 0.f};
    // visit order j = ks * MT + mt; fragment index mt * KS + ks
    v4u fb[2][FB];
#pragma unroll
    for (int j = 0; j < FB; ++j) fb[0][j] = Lk[((j % MT) * KS + j / MT) * 64];
#pragma unroll
    for (int b = 0; b < KF / FB; ++b) {
      if (b + 1 < KF / FB) {
#pragma unroll
        for (int j = 0; j < FB; ++j) {
          const int f = (b + 1) * FB + j;
          fb[(b + 1) & 1][j] = Lk[((f % MT) * KS + f / MT) * 64];
        }
      }
#pragma unroll
      for (int j = 0; j < FB; ++j) {
        const int f = b * FB + j, ks = f / MT, mt = f % MT;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          Sx[mt][nt] = mfma16(as_bf(fb[b & 1][j]), qb[nt][ks], Sx[mt][nt]);
      }
    }
  };

  auto mask = [&](int v, v4f (&Sx)[MT][NT]) {
    const int kabs0 = v * BK + 8 * a;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (kabs0 + 4 * mt + i > cpos[nt]) Sx[mt][nt][i] = -INFINITY;
  };

  auto softmax = [&](v4f (&Sx)[MT][NT], v8bf (&P)[NT], float (&alpha)[NT]) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      float mx = fmaxf(fmaxf(fmaxf(Sx[0][nt][0], Sx[0][nt][1]), fmaxf(Sx[0][nt][2], Sx[0][nt][3])),
                       fmaxf(fmaxf(Sx[1][nt][0], Sx[1][nt][1]), fmaxf(Sx[1][nt][2], Sx[1][nt][3])));
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      float mu = m_run[nt];
      if (mx > mu + thr) mu = mx;
      alpha[nt] = mu == m_run[nt] ? 1.f : __builtin_amdgcn_exp2f((m_run[nt] - mu) * c);
      m_run[nt] = mu;
      const float mc = mu == -INFINITY ? 0.f : mu * c;
      float ps = 0.f;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(Sx[mt][nt][i], c, -mc));
          Sx[mt][nt][i] = p;
          ps += p;
        }
      l_run[nt] = l_run[nt] * alpha[nt] + ps;
      v4u x;
      x[0] = pack_bf2(Sx[0][nt][0], Sx[0][nt][1]);
      x[1] = pack_bf2(Sx[0][nt][2], Sx[0][nt][3]);
      x[2] = pack_bf2(Sx[1][nt][0], Sx[1][nt][1]);
      x[3] = pack_bf2(Sx[1][nt][2], Sx[1][nt][3]);
      // Materialise P here, beside the QK MFMAs, rather than letting it sink
      // next to the P.V MFMAs that depend on it.
      asm volatile("" : "+v"(x));
      P[nt] = as_bf(x);
    }
  };

  auto pv = [&](int vslot, v8bf (&P)[NT]) {
    const lds_v4u* Lv = lane_base(Vb3, vslot);  // fragment md at Lv[md * 64]
    v4u fb[2][FB];
#pragma unroll
    for (int j = 0; j < FB; ++j) fb[0][j] = Lv[j * 64];
#pragma unroll
    for (int b = 0; b < VF / FB; ++b) {
      if (b + 1 < VF / FB) {
#pragma unroll
        for (int j = 0; j < FB; ++j) fb[(b + 1) & 1][j] = Lv[((b + 1) * FB + j) * 64];
      }
#pragma unroll
      for (int j = 0; j < FB; ++j) {
        const int md = b * FB + j;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) o[md][nt] = mfma16(as_bf(fb[b & 1][j]), P[nt], o[md][nt]);
      }
    }
  };

  // One step: issue the loads two (bf16) or one (fp8) steps ahead; S(v+1)
  // on the matrix cores alongside softmax(v) on the VALU; O += V(v) P(v);
  // then wait for the next step's tiles and release this step's slots.
  auto step = [&](int v, v4f (&Sc)[MT][NT], v4f (&Sn)[MT][NT]) {
    int issued = 0;
    int vk = -1, vv = -1;
    if (KV == 0) {
      if (v + 2 < n_st) { dma_v(v + 2); issued = 1; }
      if (v + 3 < n_st) { dma_k(v + 3); issued = 2; }
    } else {
      vk = v + 2 < n_st ? v + 2 : -1;
      vv = v + 1 < n_st ? v + 1 : -1;
      issue_fp8(vk, vv);
    }
    if (wave_active) {
      if (v * BK + BK - 1 > pos_first) mask(v, Sc);
      v8bf P[NT];
      float alpha[NT];
      qk(((v + 1) % NSLOT) * KSLOT, Sn);  // K(v+1), or stale data past the end (unused)
      softmax(Sc, P, alpha);
      bool moved = false;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) moved |= alpha[nt] != 1.f;
      if (__any(moved)) {
#pragma unroll
        for (int md = 0; md < MD; ++md)
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) o[md][nt] *= alpha[nt];
      }
      pv((v % NSLOT) * VSLOT, P);
    }
    if (KV == 0) {
      if (issued == 2) wait_vmem<KPW + VPW>();
      else if (issued == 1) wait_vmem<VPW>();
      else wait_vmem<0>();
    } else {
      commit_fp8(vk, vv);
    }
    lds_barrier();
    if (KV == 0 && v + 1 < n_st && (v + 1) * BK + BK > n_keys_t) {
      zero_tail_bf16(v + 1);
      lds_barrier();
    }
  };

  // Prologue: K(0), V(0), K(1) resident (bf16 also has K(2), V(1) in
  // flight); S(0) computed; then the slot of K(0) may be reused.
  v4f S0[MT][NT], S1[MT][NT];
  if (KV == 0) {
    dma_k(0);
    dma_v(0);
    if (n_st > 1) dma_k(1);
    if (n_st > 1) dma_v(1);
    if (n_st > 2) dma_k(2);
    if (n_st > 2) wait_vmem<KPW + VPW>();
    else if (n_st > 1) wait_vmem<VPW>();
    else wait_vmem<0>();
  } else {
    issue_fp8(0, 0);
    commit_fp8(0, 0);
    if (n_st > 1) {
      issue_fp8(1, -1);
      commit_fp8(1, -1);
    }
  }
  __syncthreads();
  if (KV == 0 && BK > n_keys_t) {
    zero_tail_bf16(0);
    __syncthreads();
  }
  if (wave_active) qk(0, S0);  // slot 0 holds K(0)
  __syncthreads();

  for (int v = 0; v < n_st; ++v) {
    step(v, S0, S1);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) S0[mt][nt] = S1[mt][nt];
  }

  if (!wave_active) return;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    float l = l_run[nt];
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    const float f = bad ? __builtin_nanf("") : A.v_scale / l;
    if (!cok[nt]) continue;
    uint16_t* dst =
        A.out + ((int64_t)(S.row_offset + crow[nt]) * A.n_q_heads + chead[nt]) * D + 4 * a;
#pragma unroll
    for (int md = 0; md < MD; ++md) {
      const v4f x = o[md][nt] * f;
      v2u w;
      w[0] = pack_bf2(x[0], x[1]);
      w[1] = pack_bf2(x[2], x[3]);
      *reinterpret_cast<v2u*>(dst + 16 * md) = w;
    }
  }
}

template <int KV, int D>
static int launch_prefill_t(const PrefillArgs& A, hipStream_t st) {
  dim3 grid((unsigned)(A.total_tiles * A.cache.n_kv_heads * (A.group / A.heads_per_wg)));
  hipLaunchKernelGGL((prefill_kernel<KV, D>), grid, dim3(256), 0, st, A);
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

int prefill_columns(int head_dim) { return 16 * prefill_ntiles(head_dim); }

int launch_prefill(const PrefillArgs& A, int kv_dtype, int head_dim, hipStream_t st) {
  if (kv_dtype == 0 && head_dim == 128) return launch_prefill_t<0, 128>(A, st);
  if (kv_dtype == 0 && head_dim == 256) return launch_prefill_t<0, 256>(A, st);
  if (kv_dtype == 1 && head_dim == 128) return launch_prefill_t<1, 128>(A, st);
  if (kv_dtype == 1 && head_dim == 256) return launch_prefill_t<1, 256>(A, st);
  return -7;
}

}  // namespace pa
