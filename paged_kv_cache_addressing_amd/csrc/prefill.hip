// Causal prompt-chunk prefill over a paged (or slab) prefix for gfx950.
//
// The prompt rows read the cache through the page table, with the page size
// a compile-time constant of 256 and one page lookup per page (TensorFold
// pull request #1373, prompt rows; pull request #2011, hpattn_p256_kernel and
// "a paged item's page looked up once").  Keys past a row's limit land as
// zeros (pull request #2011 review, "Is paged output the same as windowed
// output?").
//
// One workgroup = 4 waves = 128 query rows of one stream x one q head; each
// wave owns 32 rows (two 16-column MFMA n-tiles).  Key tiles of 64 keys are
// staged HBM -> registers -> LDS, double buffered, in "fragment order": the
// 1 KiB a wave reads for one MFMA operand is contiguous in LDS (lane l's 16
// bytes at l*16), so every ds_read_b128 is conflict-free.  fp8 tiles are
// converted to bf16 once, while staging.
//   S^T (64 keys x 32 rows) = K Q^T     : 4 m-tiles x 2 n-tiles x D/32 k-steps
//   O^T (D x 32 rows)      += V^T P^T   : D/16 m-tiles x 2 n-tiles x 2 k-steps
// The key order inside a tile is permuted so each lane's S^T C-rows are the
// 8 consecutive keys of its P^T operand (no shuffles between the products).
//
// Row independence: a row's arithmetic depends only on its own position
// and the keys; key tiles run from 0 in fixed order, and a tile that is
// wholly masked for a row leaves its state bit-identical (alpha = 2^0 = 1,
// p = 0 against finite or zeroed values).  So splitting a stream's rows
// across calls gives the same bytes as one call.
#include "pa_device.hpp"
#include "pa_internal.hpp"

namespace pa {

template <int KV, int D>
__global__ __launch_bounds__(256, 1) void prefill_kernel(const PrefillArgs A) {
  constexpr int ESZ = KV ? 1 : 2;
  constexpr int BK = 64;             // keys per tile
  constexpr int MT = 4;              // S^T m-tiles per key tile
  constexpr int KKT = 2;             // PV k-steps per key tile
  constexpr int KS = D / 32;         // QK k-steps
  constexpr int MD = D / 16;         // O^T m-tiles
  constexpr int NT = 2;              // n-tiles (16 rows) per wave
  constexpr int KF = MT * KS;        // K fragments (1 KiB each) per tile
  constexpr int VF = MD * KKT;       // V fragments per tile
  constexpr int FR = (KF + VF) * 64; // 16-byte LDS entries per buffer
  constexpr int KLD = KV ? KF * 64 / 2 / 256 : KF * 64 / 256;  // staging loads / thread
  constexpr int VLD = KV ? MD * 64 / 256 : VF * 64 / 256;
  static_assert(kPage % BK == 0, "a key tile never straddles two pages");

  __shared__ v4u lds[2 * FR];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int n = lane & 15;
  const int a = lane >> 4;
  const int head = blockIdx.x % A.n_q_heads;
  const int tg = A.total_tiles - 1 - (int)(blockIdx.x / A.n_q_heads);  // longest tiles first
  const int si = find_stream<0>(A.s, A.n_streams, tg);
  const StreamArg& S = A.s[si];
  const int row0 = (tg - S.block_begin) * kPrefillRows;
  const int rows_here = min(kPrefillRows, S.n_rows - row0);
  const int pos_first = S.first_pos + row0;
  const int pos_last = pos_first + rows_here - 1;
  const int n_keys_t = pos_last + 1;
  const int n_kt = (n_keys_t + BK - 1) / BK;
  const int g = head / A.group;
  const bool wave_active = 32 * wave < rows_here;

  int rr[NT], pos[NT];
  bool ok[NT];
  v8bf qb[NT][KS];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    rr[nt] = row0 + 32 * wave + 16 * nt + n;
    ok[nt] = rr[nt] < row0 + rows_here;
    pos[nt] = ok[nt] ? S.first_pos + rr[nt] : pos_last;
    const uint8_t* qp = reinterpret_cast<const uint8_t*>(A.q) +
                        ((int64_t)(S.row_offset + (ok[nt] ? rr[nt] : row0)) * A.n_q_heads + head) *
                            D * 2;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int d0 = KV ? 64 * (ks >> 1) + 16 * a + 8 * (ks & 1) : 32 * ks + 8 * a;
      v4u x = load16(qp + d0 * 2);
      if (!ok[nt]) x = v4u{0, 0, 0, 0};
      qb[nt][ks] = as_bf(x);
    }
  }

  v4u st_k[KLD], st_v[VLD];
  PageTile T{};
  bool bad = false;

  // Global -> registers for key tile u (the page is looked up once per page).
  auto issue = [&](int u) {
    if ((u & 3) == 0) {
      T = page_tile<D, ESZ>(S, A.cache, u >> 2, g);
      bad |= !T.ok;
    }
    const int o = (u & 3) * BK;
#pragma unroll
    for (int i = 0; i < KLD; ++i) {
      const int q = i * 256 + tid;
      const int lp = q & 63;
      const int m = lp & 15;
      const int key = 16 * (m >> 2) + (m & 3);
      if (KV) {
        const int fp = q >> 6;
        const int mt = fp / (KS / 2), kq = fp % (KS / 2);
        st_k[i] = load16(T.k + (int64_t)(o + key + 4 * mt) * D + 64 * kq + 16 * (lp >> 4));
      } else {
        const int f = q >> 6;
        const int mt = f / KS, ks = f % KS;
        st_k[i] = load16(T.k + ((int64_t)(o + key + 4 * mt) * D + 32 * ks + 8 * (lp >> 4)) * 2);
      }
    }
#pragma unroll
    for (int i = 0; i < VLD; ++i) {
      const int q = i * 256 + tid;
      const int lp = q & 63;
      if (KV) {
        const int md = q >> 6;
        const int d = 16 * md + (lp & 15);
        st_v[i] = load16(T.v + v_off<D, ESZ>(o + 16 * (lp >> 4), d));
      } else {
        const int f = q >> 6;
        const int md = f >> 1, kk = f & 1;
        const int d = 16 * md + (lp & 15);
        st_v[i] = load16(T.v + v_off<D, ESZ>(o + 16 * (lp >> 4) + 8 * kk, d) * 2);
      }
    }
  };

  // Registers -> LDS buffer, converting fp8 and zeroing values past the limit.
  auto commit = [&](int u, int buf) {
    v4u* L = lds + buf * FR;
    const bool tail = u * BK + BK > n_keys_t;
#pragma unroll
    for (int i = 0; i < KLD; ++i) {
      const int q = i * 256 + tid;
      const int lp = q & 63;
      if (KV) {
        const int fp = q >> 6;
        const int mt = fp / (KS / 2), kq = fp % (KS / 2);
        const int f0 = mt * KS + 2 * kq;
        L[f0 * 64 + lp] = __builtin_bit_cast(v4u, fp8x8_to_bf16(st_k[i][0], st_k[i][1]));
        L[(f0 + 1) * 64 + lp] = __builtin_bit_cast(v4u, fp8x8_to_bf16(st_k[i][2], st_k[i][3]));
      } else {
        L[q] = st_k[i];
      }
    }
#pragma unroll
    for (int i = 0; i < VLD; ++i) {
      const int q = i * 256 + tid;
      const int lp = q & 63;
      if (KV) {
        const int md = q >> 6;
        v4u x = st_v[i];
        if (tail) x = keep_first_b(x, n_keys_t - (u * BK + 16 * (lp >> 4)));
        const int f0 = KF + 2 * md;
        L[f0 * 64 + lp] = __builtin_bit_cast(v4u, fp8x8_to_bf16(x[0], x[1]));
        L[(f0 + 1) * 64 + lp] = __builtin_bit_cast(v4u, fp8x8_to_bf16(x[2], x[3]));
      } else {
        const int kk = (q >> 6) & 1;
        v4u x = st_v[i];
        if (tail) x = keep_first_h(x, n_keys_t - (u * BK + 16 * (lp >> 4) + 8 * kk));
        L[KF * 64 + q] = x;
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

  issue(0);
  commit(0, 0);
  __syncthreads();

  for (int u = 0; u < n_kt; ++u) {
    if (u + 1 < n_kt) issue(u + 1);
    if (wave_active) {
      const v4u* L = lds + (u & 1) * FR;
      v4f sacc[MT][NT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) sacc[mt][nt] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const v8bf ka = as_bf(L[(mt * KS + ks) * 64 + lane]);
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) sacc[mt][nt] = mfma16(ka, qb[nt][ks], sacc[mt][nt]);
        }

      const bool need_mask = u * BK + BK - 1 > pos_first;
      const int kabs0 = u * BK + 16 * a;
      float alpha[NT];
      v8bf pb[NT][KKT];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        float sv[MT][4];
        float mx = -INFINITY;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float v = sacc[mt][nt][i] * A.scale_log2;
            if (need_mask && kabs0 + 4 * mt + i > pos[nt]) v = -INFINITY;
            sv[mt][i] = v;
            mx = fmaxf(mx, v);
          }
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(m_run[nt], mx);
        const float m_use = m_new == -INFINITY ? 0.f : m_new;
        alpha[nt] = __builtin_amdgcn_exp2f(m_run[nt] - m_use);
        float psum = 0.f;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            sv[mt][i] = __builtin_amdgcn_exp2f(sv[mt][i] - m_use);
            psum += sv[mt][i];
          }
        l_run[nt] = l_run[nt] * alpha[nt] + psum;
        m_run[nt] = m_new;
#pragma unroll
        for (int kk = 0; kk < KKT; ++kk) {
          v4u x;
          x[0] = pack_bf2(sv[2 * kk][0], sv[2 * kk][1]);
          x[1] = pack_bf2(sv[2 * kk][2], sv[2 * kk][3]);
          x[2] = pack_bf2(sv[2 * kk + 1][0], sv[2 * kk + 1][1]);
          x[3] = pack_bf2(sv[2 * kk + 1][2], sv[2 * kk + 1][3]);
          pb[nt][kk] = as_bf(x);
        }
      }
      if (__any(alpha[0] != 1.f || alpha[1] != 1.f)) {
#pragma unroll
        for (int md = 0; md < MD; ++md)
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) o[md][nt] *= alpha[nt];
      }
#pragma unroll
      for (int md = 0; md < MD; ++md)
#pragma unroll
        for (int kk = 0; kk < KKT; ++kk) {
          const v8bf va = as_bf(L[(KF + md * KKT + kk) * 64 + lane]);
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) o[md][nt] = mfma16(va, pb[nt][kk], o[md][nt]);
        }
    }
    if (u + 1 < n_kt) commit(u + 1, (u + 1) & 1);
    __syncthreads();
  }

  if (!wave_active) return;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    float l = l_run[nt];
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    const float f = bad ? __builtin_nanf("") : A.v_scale / l;
    if (!ok[nt]) continue;
    uint16_t* dst = A.out + ((int64_t)(S.row_offset + rr[nt]) * A.n_q_heads + head) * D + 4 * a;
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
  dim3 grid((unsigned)(A.total_tiles * A.n_q_heads));
  hipLaunchKernelGGL((prefill_kernel<KV, D>), grid, dim3(256), 0, st, A);
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

int launch_prefill(const PrefillArgs& A, int kv_dtype, int head_dim, hipStream_t st) {
  if (kv_dtype == 0 && head_dim == 128) return launch_prefill_t<0, 128>(A, st);
  if (kv_dtype == 0 && head_dim == 256) return launch_prefill_t<0, 256>(A, st);
  if (kv_dtype == 1 && head_dim == 128) return launch_prefill_t<1, 128>(A, st);
  if (kv_dtype == 1 && head_dim == 256) return launch_prefill_t<1, 256>(A, st);
  return -7;
}

}  // namespace pa
