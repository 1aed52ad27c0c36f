// Split-K paged decode for gfx950: partial kernel (MFMA) + log-sum-exp merge.
//
// Decode is a split partial followed by a merge (TensorFold issue #1344,
// "Mechanism"); the decode tiles read key rows through the page table, one
// lookup per page (pull request #2011, "What this changes").  One workgroup
// owns splits_per_wg consecutive 4096-key splits of one (stream, kv head,
// 16-column tile); its four waves take each split's pages round-robin and
// are combined in fixed wave order, so the partial of a split depends on
// that split's keys and queries alone, whichever workgroup computes it.
//
// MFMA mapping (v_mfma_f32_16x16x32_bf16, wave64):
//   S^T = K Q^T : A = 16 keys x 32 dims of K, B = 32 dims x 16 columns of Q^T,
//                 a column being one (query row, q head of the group).
//   O^T += V^T P^T : A = 16 dims x 32 keys of V^T (V is dim-major inside
//                 64-byte key blocks, so a lane's 8 keys are one 16-byte
//                 load and a chunk's V is one contiguous run), B = P^T.
// The keys of each S^T m-tile are permuted so that the C-layout rows a lane
// ends up holding are exactly the 8 consecutive keys its P^T operand needs:
// no data moves between the two products.  K and V go straight from HBM to
// registers: with one column tile no operand is shared across waves, so
// staging through LDS would add latency and no reuse.
#include "pa_device.hpp"
#include "pa_internal.hpp"

namespace pa {

// First dim of the 8-dim run a lane of lane-group `a` holds at QK k-step ks.
// bf16: natural order.  fp8: two k-steps share one 16-byte load, so the run
// for (ks, a) is dims 64*(ks/2) + 16a + 8*(ks%2) .. +7.  Q^T follows the same
// permutation, so the dot product is unchanged.
template <int KV>
__device__ __forceinline__ int qk_d(int ks, int a) {
  return KV ? (64 * (ks >> 1) + 16 * a + 8 * (ks & 1)) : (32 * ks + 8 * a);
}

template <int KV, int D, bool DIRECT>
__global__ __launch_bounds__(256, 1) void decode_partial_kernel(const DecodeArgs A) {
  constexpr int ESZ = KV ? 1 : 2;
  constexpr int KK = KV ? 2 : 1;      // 32-key PV k-steps per chunk
  constexpr int CK = 32 * KK;         // keys per chunk
  constexpr int MT = 2 * KK;          // 16-key S^T m-tiles per chunk
  constexpr int KS = D / 32;          // QK k-steps
  constexpr int MD = D / 16;          // O^T m-tiles
  constexpr int NW = 4;               // waves per workgroup
  constexpr int KL = KV ? MT * KS / 2 : MT * KS;  // 16-byte K loads per lane per chunk

  // Wave states at the end of a split, double-buffered by split parity.
  constexpr int MQ = MD / NW;  // O^T m-tiles each wave merges and writes
  __shared__ v4f sh_o[2][NW][MD][64];
  __shared__ float sh_m[2][NW][64];
  __shared__ float sh_l[2][NW][64];
  __shared__ int sh_bad[2][NW];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform: SGPR arithmetic
  const int n = lane & 15;
  const int a = lane >> 4;
  const int g = blockIdx.y;
  const int ct = blockIdx.x % A.col_tiles;
  const int item = blockIdx.x / A.col_tiles;
  const int si = find_stream<0>(A.s, A.n_streams, item);
  const StreamArg& S = A.s[si];
  const int split0 = (item - S.block_begin) * A.splits_per_wg;  // first split of the workgroup
  const int n_sub = min(A.splits_per_wg, S.n_splits - split0);
  const int G = A.group;
  if (16 * ct >= G * S.n_rows) return;  // tile holds no column of this stream

  const int col = 16 * ct + n;
  const int r = col / G;
  const int hl = col - r * G;
  const bool col_ok = r < S.n_rows;
  const int pos = col_ok ? S.first_pos + r : S.n_keys - 1;
  const int h = g * G + hl;
  // Visible keys of the column's row: all up to pos; with an ancestor table,
  // of the rows' own keys first_pos + j only those whose bit j is set.
  const uint32_t anc = (S.tree_mask && col_ok) ? S.tree_mask[r] : 0xFFFFFFFFu;
  const int mask_from = S.tree_mask ? S.first_pos : S.first_pos + 1;  // first maskable key

  v8bf qb[KS];
  {
    const uint8_t* qp = reinterpret_cast<const uint8_t*>(A.q) +
                        ((int64_t)(S.row_offset + (col_ok ? r : 0)) * A.n_q_heads + h) * D * 2;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      v4u x = load16(qp + qk_d<KV>(ks, a) * 2);
      if (!col_ok) x = v4u{0, 0, 0, 0};
      qb[ks] = as_bf(x);
    }
  }

  const int k_lo = split0 * A.split_keys;
  const int k_hi = min(k_lo + n_sub * A.split_keys, S.n_keys);
  const int p_lo = k_lo / kPage;
  const int p_hi = (k_hi + kPage - 1) / kPage;
  // Pages of a whole split.  With more than one split per workgroup the host
  // makes it a multiple of NW, so wave w meets the same pages of every split
  // (those p_lo(split) + w + NW i) as it would alone.
  const int pps = A.split_keys / kPage;
  // The split (0 .. n_sub-1) of the workgroup a page belongs to.
  auto sub = [&](int p) { return (p - p_lo) / pps; };
  // The waves walk a split's pages in the order p_lo(split) + wave, + NW,
  // ..., read through a rotation by the split index: physical page
  // p_lo(split) + (p - p_lo(split) + split) mod (pages of the split).
  // Contiguous slabs put the splits of a stream at regular strides, and
  // without it every workgroup would touch the same offsets of its split at
  // the same time.  The rotation depends on the split alone, never on the
  // batch.
  // A look-ahead may ask for a page at or past p_hi (its result is never
  // used); np is kept >= 1 there so the remainder stays defined.
  auto phys = [&](int p) {
    const int sb = sub(p);
    const int base = p_lo + sb * pps;
    const int np = max(1, min(pps, p_hi - base));
    int v = p - base + (split0 + sb) % np;
    if (v >= np) v -= np;
    return base + v;
  };

  v4f o[MD];
#pragma unroll
  for (int md = 0; md < MD; ++md) o[md] = v4f{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;
  bool bad = false;

  // S^T row m of m-tile mt holds key 8*KK*(m/4) + 4*mt + m%4 of the chunk.
  const int krow = 8 * KK * (n >> 2) + (n & 3);

  // The wave's chunks, in order: its pages p_lo + wave, + NW, ..., each cut
  // into CK-key chunks up to the split's end.  Two register sets alternate,
  // two chunks ahead: once the S^T products of chunk i have read its K
  // registers they are refilled with the K of chunk i+2, and likewise V after
  // the P.V products, so about one and a half chunks of bytes stay in flight
  // while the wave computes.  Each K/V byte is read once, so the loads are
  // streaming (nontemporal).
  auto load_k = [&](v4u (&kr)[KL], const PageTile& T, int c0) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const uint8_t* kp = T.k + (int64_t)(c0 + krow + 4 * mt) * D * ESZ;
      if (KV) {
#pragma unroll
        for (int kq = 0; kq < KS / 2; ++kq) kr[mt * (KS / 2) + kq] = load16_stream(kp + 64 * kq + 16 * a);
      } else {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) kr[mt * KS + ks] = load16_stream(kp + (32 * ks + 8 * a) * 2);
      }
    }
  };
  // V block of a chunk (CK == 64/ESZ keys): D rows of 64 bytes.
  auto load_v = [&](v4u (&vr)[MD], const PageTile& T, int c0) {
    const uint8_t* vb = T.v + (int64_t)c0 * D * ESZ + (8 * KK * a) * ESZ;
#pragma unroll
    for (int md = 0; md < MD; ++md) vr[md] = load16_stream(vb + (16 * md + n) * 64);
  };
  auto chunk = [&](v4u (&kr)[KL], v4u (&vr)[MD], int p, int c0, auto after_qk, auto after_pv) {
    v4f sacc[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      sacc[mt] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        v8bf ka;
        if (KV) {
          const v4u x = kr[mt * (KS / 2) + (ks >> 1)];
          ka = (ks & 1) ? fp8x8_to_bf16(x[2], x[3]) : fp8x8_to_bf16(x[0], x[1]);
        } else {
          ka = as_bf(kr[mt * KS + ks]);
        }
        sacc[mt] = mfma16(ka, qb[ks], sacc[mt]);
      }
    }
    after_qk();

    // Online softmax for this lane's column over its 4*MT keys.
    const int kabs0 = p * kPage + c0 + 8 * KK * a;
    const bool need_mask = p * kPage + c0 + CK - 1 >= mask_from;
    float sv[MT][4];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) sv[mt][i] = sacc[mt][i] * A.scale_log2;
    // Only chunks that reach a row's own keys can hold a masked key; the
    // test is wave-uniform, so the mask is skipped as a whole elsewhere.
    if (need_mask) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int kabs = kabs0 + 4 * mt + i, rel = kabs - S.first_pos;
          const bool vis = (kabs <= pos) & ((rel < 0) | (((anc >> (rel & 31)) & 1u) != 0u));
          sv[mt][i] = vis ? sv[mt][i] : -INFINITY;
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) mx = fmaxf(mx, sv[mt][i]);
    mx = rows4_max(mx);
    const float m_new = fmaxf(m_run, mx);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    float psum = 0.f;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sv[mt][i] = __builtin_amdgcn_exp2f(sv[mt][i] - m_use);
        psum += sv[mt][i];
      }
    l_run = l_run * alpha + psum;
    m_run = m_new;
    if (__any(alpha != 1.f)) {
#pragma unroll
      for (int md = 0; md < MD; ++md) o[md] *= alpha;
    }
    v8bf pb[KK];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      v4u x;
      x[0] = pack_bf2(sv[2 * kk][0], sv[2 * kk][1]);
      x[1] = pack_bf2(sv[2 * kk][2], sv[2 * kk][3]);
      x[2] = pack_bf2(sv[2 * kk + 1][0], sv[2 * kk + 1][1]);
      x[3] = pack_bf2(sv[2 * kk + 1][2], sv[2 * kk + 1][3]);
      pb[kk] = as_bf(x);
    }

    // Keys at or past n_keys may be unwritten: their values land as zeros.
    if (p * kPage + c0 + CK > S.n_keys) {
      const int nv = S.n_keys - kabs0;
#pragma unroll
      for (int md = 0; md < MD; ++md) vr[md] = KV ? keep_first_b(vr[md], nv) : keep_first_h(vr[md], nv);
    }
#pragma unroll
    for (int md = 0; md < MD; ++md)
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        v8bf va;
        if (KV)
          va = kk ? fp8x8_to_bf16(vr[md][2], vr[md][3]) : fp8x8_to_bf16(vr[md][0], vr[md][1]);
        else
          va = as_bf(vr[md]);
        o[md] = mfma16(va, pb[kk], o[md]);
      }
    after_pv();
  };
  // (p, c0) -> the wave's next chunk
  auto advance = [&](int& p, int& c0) {
    c0 += CK;
    if (c0 >= min(kPage, k_hi - phys(p) * kPage)) {
      p += NW;
      c0 = 0;
    }
  };
  // The end of split `done` of the workgroup: the waves' states go to the
  // LDS set of its parity and, after a barrier, each wave merges them in
  // fixed wave order for a quarter of the dims and writes that quarter of the
  // partial; every wave then starts the next split afresh.  Spreading the
  // merge keeps the stores (which the next chunk's load wait also counts)
  // and the merge arithmetic off a single wave.  The barrier only orders
  // LDS: loads of the next split already in flight stay in flight.  A wave
  // reads a set before it reaches the next barrier, so the set is free again
  // when the split after next ends.
  int done = 0;
  auto boundary = [&]() __attribute__((always_inline)) {
    const int sp = done & 1;
    // Per-column row sum across the four lane groups, in a fixed order.
    const float l_own = rows4_sum(l_run);
#pragma unroll
    for (int md = 0; md < MD; ++md) sh_o[sp][wave][md][lane] = o[md];
    sh_m[sp][wave][lane] = m_run;
    sh_l[sp][wave][lane] = l_own;
    if (lane == 0) sh_bad[sp][wave] = bad ? 1 : 0;
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    bool any_bad = false;
#pragma unroll
    for (int w = 0; w < NW; ++w) any_bad |= sh_bad[sp][w] != 0;
    // Merge the waves in fixed order 0, 1, .., NW-1; this wave takes the
    // O^T m-tiles MQ*wave .. MQ*wave+MQ-1, every wave the same (m, l).
    float m_acc = sh_m[sp][0][lane];
    float l_sum = sh_l[sp][0][lane];
    v4f acc[MQ];
#pragma unroll
    for (int j = 0; j < MQ; ++j) acc[j] = sh_o[sp][0][MQ * wave + j][lane];
    for (int w = 1; w < NW; ++w) {
      const float mw = sh_m[sp][w][lane];
      const float lw = sh_l[sp][w][lane];
      const float M = fmaxf(m_acc, mw);
      if (M == -INFINITY) continue;
      const float a0 = __builtin_amdgcn_exp2f(m_acc - M);
      const float aw = __builtin_amdgcn_exp2f(mw - M);
#pragma unroll
      for (int j = 0; j < MQ; ++j) acc[j] = acc[j] * a0 + sh_o[sp][w][MQ * wave + j][lane] * aw;
      l_sum = l_sum * a0 + lw * aw;
      m_acc = M;
    }
    if constexpr (DIRECT) {
      if (col_ok) {
        // The call's only split: the merge would weigh it by 2^(m - m) = 1,
        // so its result is o / l * v_scale, computed here in the merge's
        // operation order (the same bytes) without the partials' round trip.
        uint16_t* dst = A.out + ((int64_t)(S.row_offset + r) * A.n_q_heads + h) * D + 4 * a;
#pragma unroll
        for (int j = 0; j < MQ; ++j)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            dst[16 * (MQ * wave + j) + e] = f2bf(any_bad ? __builtin_nanf("") : acc[j][e] / l_sum * A.v_scale);
      }
    } else if (col_ok) {
      const int64_t slot =
          S.slot_base + ((int64_t)r * A.n_q_heads + h) * S.n_splits + split0 + done;
      if (wave == 0 && a == 0) {
        A.ws_ml[2 * slot] = any_bad ? __builtin_nanf("") : m_acc;
        A.ws_ml[2 * slot + 1] = l_sum;
      }
      float* dst = A.ws_o + slot * D + 4 * a;
#pragma unroll
      for (int j = 0; j < MQ; ++j) *reinterpret_cast<v4f*>(dst + 16 * (MQ * wave + j)) = acc[j];
    }
#pragma unroll
    for (int md = 0; md < MD; ++md) o[md] = v4f{0.f, 0.f, 0.f, 0.f};
    m_run = -INFINITY;
    l_run = 0.f;
    bad = false;
    ++done;
  };

  // Chunks i (p0, c0), i+1 (p1, c1) and i+2 (p2, c2), with their page tiles;
  // the page table is read once per page as a chunk first enters the queue.
  v4u krA[KL], vrA[MD], krB[KL], vrB[MD];
  int p0 = p_lo + wave, c0 = 0;
  int p1 = p0, c1 = c0;
  advance(p1, c1);
  PageTile T0{}, T1{};
  if (p0 < p_hi) {
    T0 = page_tile<D, ESZ>(S, A.cache, phys(p0), g);
    bad |= !T0.ok;
    load_k(krA, T0, c0);
    load_v(vrA, T0, c0);
  }
  if (p1 < p_hi) {
    T1 = T0;
    if (p1 != p0) {
      T1 = page_tile<D, ESZ>(S, A.cache, phys(p1), g);
      bad |= !T1.ok;
    }
    load_k(krB, T1, c1);
    load_v(vrB, T1, c1);
  }
  // Compute chunk i from (kr, vr), refilling them with chunk i+2.
  auto run_chunk = [&](v4u (&kr)[KL], v4u (&vr)[MD]) {
    int p2 = p1, c2 = c1;
    advance(p2, c2);
    PageTile T2 = T1;
    const bool more = p2 < p_hi;
    if (more && p2 != p1) {
      T2 = page_tile<D, ESZ>(S, A.cache, phys(p2), g);
      bad |= !T2.ok;
    }
    chunk(kr, vr, phys(p0), c0, [&] { if (more) load_k(kr, T2, c2); },
          [&] { if (more) load_v(vr, T2, c2); });
    p0 = p1;
    c0 = c1;
    T0 = T1;
    p1 = p2;
    c1 = c2;
    T1 = T2;
    // the splits this wave has finished (its next chunk lies beyond them)
    const int s_next = p0 < p_hi ? sub(p0) : n_sub;
    while (done < s_next) boundary();
  };
  while (p0 < p_hi) {
    run_chunk(krA, vrA);
    if (p0 >= p_hi) break;
    run_chunk(krB, vrB);
  }

  while (done < n_sub) boundary();
}

// out[row][h] = v_scale * sum_j 2^(m_j - M) o_j / sum_j 2^(m_j - M) l_j, in
// split order j = 0, 1, ...; a wholly masked split (m_j = -inf) weighs 0.
// One wave per (row, q head), lane l owning dims DV*l .. DV*l+DV-1 (16-byte
// loads at D = 256).  Lane j holds the weight 2^(m_j - M) and l_j of split
// j of the current run of 64; every lane reads them with readlane, so no
// value goes through LDS and there is no barrier.  The first JB splits' o_j
// go out with the (m_j, l_j) loads.  All sums run in split order, so the
// result does not depend on how the splits are batched.
template <int D>
__global__ __launch_bounds__(64) void decode_merge_kernel(const DecodeArgs A) {
  constexpr int DV = D / 64;  // dims per lane
  constexpr int JB = 16;      // splits of o_j loads in flight
  typedef float vdf __attribute__((ext_vector_type(DV)));
  const int row = blockIdx.x;
  const int h = blockIdx.y;
  const int lane = threadIdx.x;
  const int si = find_stream_wave<1>(A.s, A.n_streams, row);
  const StreamArg& S = A.s[si];
  const int r = row - S.row_begin;
  const int ns = S.n_splits;
  const int64_t slot0 = S.slot_base + ((int64_t)r * A.n_q_heads + h) * ns;
  const float* ml = A.ws_ml + 2 * slot0;
  const vdf* op = reinterpret_cast<const vdf*>(A.ws_o + slot0 * D) + lane;

  vdf o0[JB];
#pragma unroll
  for (int u = 0; u < JB; ++u) o0[u] = u < ns ? op[(int64_t)u * (D / DV)] : vdf{};
  const float m_t = lane < ns ? ml[2 * lane] : -INFINITY;
  const float l_t = lane < ns ? ml[2 * lane + 1] : 0.f;

  // M = max_j m_j (exact in any order); a NaN m marks a rejected page id.
  float mx = m_t;
  bool bad = m_t != m_t;
  for (int j = lane + 64; j < ns; j += 64) {
    const float m = ml[2 * j];
    bad |= m != m;
    mx = fmaxf(mx, m);
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
  const bool any_bad = __any(bad);
  const float M = mx;

  vdf num = vdf{};
  float den = 0.f;
  for (int j0 = 0; j0 < ns; j0 += 64) {
    const int nj = min(64, ns - j0);
    float wj = 0.f, lj = 0.f;
    if (lane < nj) {
      const float m = j0 == 0 ? m_t : ml[2 * (j0 + lane)];
      wj = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m - M);
      lj = j0 == 0 ? l_t : ml[2 * (j0 + lane) + 1];
    }
    for (int jb = 0; jb < nj; jb += JB) {
      vdf ob[JB];
      if (j0 == 0 && jb == 0) {
#pragma unroll
        for (int u = 0; u < JB; ++u) ob[u] = o0[u];
      } else {
#pragma unroll
        for (int u = 0; u < JB; ++u)
          ob[u] = jb + u < nj ? op[(int64_t)(j0 + jb + u) * (D / DV)] : vdf{};
      }
#pragma unroll
      for (int u = 0; u < JB; ++u) {
        if (jb + u >= nj) break;
        const float w = __builtin_bit_cast(float, __builtin_amdgcn_readlane(
                                                      __builtin_bit_cast(int, wj), jb + u));
        const float l = __builtin_bit_cast(float, __builtin_amdgcn_readlane(
                                                      __builtin_bit_cast(int, lj), jb + u));
#pragma unroll
        for (int d = 0; d < DV; ++d) num[d] += w * ob[u][d];
        den += w * l;
      }
    }
  }
  uint16_t* dst = A.out + ((int64_t)(S.row_offset + r) * A.n_q_heads + h) * D + DV * lane;
#pragma unroll
  for (int d = 0; d < DV; ++d) dst[d] = f2bf(any_bad ? __builtin_nanf("") : num[d] / den * A.v_scale);
}

template <int KV, int D>
static int launch_partials_t(const DecodeArgs& A, int n_kv_heads, hipStream_t st) {
  dim3 grid((unsigned)(A.total_items * A.col_tiles), (unsigned)n_kv_heads);
  // the direct-output form is its own instance, so the partial-writing one
  // is compiled exactly as without it
  if (A.direct_out)
    hipLaunchKernelGGL((decode_partial_kernel<KV, D, true>), grid, dim3(256), 0, st, A);
  else
    hipLaunchKernelGGL((decode_partial_kernel<KV, D, false>), grid, dim3(256), 0, st, A);
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

int launch_decode_partials(const DecodeArgs& A, int kv_dtype, int head_dim, int n_kv_heads,
                           hipStream_t st) {
  if (kv_dtype == 0 && head_dim == 128) return launch_partials_t<0, 128>(A, n_kv_heads, st);
  if (kv_dtype == 0 && head_dim == 256) return launch_partials_t<0, 256>(A, n_kv_heads, st);
  if (kv_dtype == 1 && head_dim == 128) return launch_partials_t<1, 128>(A, n_kv_heads, st);
  if (kv_dtype == 1 && head_dim == 256) return launch_partials_t<1, 256>(A, n_kv_heads, st);
  return -7;
}

int launch_decode_merge(const DecodeArgs& A, int head_dim, hipStream_t st) {
  dim3 grid((unsigned)A.total_rows, (unsigned)A.n_q_heads);
  if (head_dim == 128)
    hipLaunchKernelGGL((decode_merge_kernel<128>), grid, dim3(64), 0, st, A);
  else if (head_dim == 256)
    hipLaunchKernelGGL((decode_merge_kernel<256>), grid, dim3(64), 0, st, A);
  else
    return -7;
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

}  // namespace pa
