// KV store for gfx950: scatter new key/value rows into their pages (or slab),
// quantising to E4M3FN for fp8 caches.  The layout written is the one every
// attention kernel reads (TensorFold pull request #1373, "What changes": the
// tiles read the layout the stores write): K head-major [g][slot][D] and V
// in 64-byte key blocks, dim-major inside a block, [g][slot/VB][D][slot%VB].
#include "pa_device.hpp"
#include "pa_internal.hpp"

namespace pa {

// RNE_E4M3FN(clamp(fl32(x / scale), -448, 448)); NaN -> 0x7F.
__device__ __forceinline__ uint32_t enc_e4m3(float x, float scale) {
  float y = x / scale;
  if (y != y) return 0x7Fu;
  y = fminf(fmaxf(y, -448.f), 448.f);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(y, y, 0, false) & 0xFFu;
}

__device__ __forceinline__ float bf2f(uint16_t b) {
  return __builtin_bit_cast(float, (uint32_t)b << 16);
}

// One block per (row, kv head); thread d stores dim d of K and of V.
template <int KV, int D>
__global__ __launch_bounds__(256) void write_kv_kernel(const WriteArgs A) {
  constexpr int ESZ = KV ? 1 : 2;
  const int row = blockIdx.x;
  const int g = blockIdx.y;
  const int si = find_stream_wave<1>(A.s, A.n_streams, row);
  const StreamArg& S = A.s[si];
  const int r = row - S.row_begin;
  const int pos = S.first_pos + r;
  // The new row's values do not depend on the page: their loads go out
  // before the page-table read, so the two latencies overlap.  The grid
  // gives one thread per dim (blockDim.x == D).
  const int d = threadIdx.x;
  const int64_t src = ((int64_t)(S.row_offset + r) * A.cache.n_kv_heads + g) * D;
  const uint16_t kx = A.k_new[src + d];
  const uint16_t vx = A.v_new[src + d];
  const PageTile T = page_tile<D, ESZ>(S, A.cache, pos / kPage, g);
  if (!T.ok) return;
  const int j = pos % kPage;
  {
    uint8_t* kd = T.k + ((int64_t)j * D + d) * ESZ;
    uint8_t* vd = T.v + (int64_t)v_off<D, ESZ>(j, d) * ESZ;
    if (KV) {
      *kd = (uint8_t)enc_e4m3(bf2f(kx), A.k_scale);
      *vd = (uint8_t)enc_e4m3(bf2f(vx), A.v_scale);
    } else {
      *reinterpret_cast<uint16_t*>(kd) = kx;
      *reinterpret_cast<uint16_t*>(vd) = vx;
    }
  }
}

template <int KV, int D>
static int launch_write_t(const WriteArgs& A, hipStream_t st) {
  dim3 grid((unsigned)A.total_rows, (unsigned)A.cache.n_kv_heads);
  hipLaunchKernelGGL((write_kv_kernel<KV, D>), grid, dim3(D), 0, st, A);
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

int launch_write_kv(const WriteArgs& A, int kv_dtype, int head_dim, hipStream_t st) {
  if (kv_dtype == 0 && head_dim == 128) return launch_write_t<0, 128>(A, st);
  if (kv_dtype == 0 && head_dim == 256) return launch_write_t<0, 256>(A, st);
  if (kv_dtype == 1 && head_dim == 128) return launch_write_t<1, 128>(A, st);
  if (kv_dtype == 1 && head_dim == 256) return launch_write_t<1, 256>(A, st);
  return -7;
}

}  // namespace pa
