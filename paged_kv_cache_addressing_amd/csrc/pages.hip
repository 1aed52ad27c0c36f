// Whole-page device copies (copy on write of shared prefix pages).  One
// workgroup row per (src, dst) pair; each thread moves 16 bytes per
// iteration with plain vector loads and stores.
#include "pa_internal.hpp"

namespace pa {

__global__ __launch_bounds__(256) void page_copy_kernel(const PageCopyArgs A) {
  const int pair = blockIdx.y;
  const int64_t chunks = A.page_bytes / 16;
  const uint8_t* ks = A.k + (int64_t)A.src[pair] * A.page_bytes;
  const uint8_t* vs = A.v + (int64_t)A.src[pair] * A.page_bytes;
  uint8_t* kd = A.k + (int64_t)A.dst[pair] * A.page_bytes;
  uint8_t* vd = A.v + (int64_t)A.dst[pair] * A.page_bytes;
  typedef uint32_t v4u __attribute__((__vector_size__(16)));
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < chunks;
       i += (int64_t)gridDim.x * blockDim.x) {
    reinterpret_cast<v4u*>(kd)[i] = reinterpret_cast<const v4u*>(ks)[i];
    reinterpret_cast<v4u*>(vd)[i] = reinterpret_cast<const v4u*>(vs)[i];
  }
}

int launch_page_copy(const PageCopyArgs& A, hipStream_t st) {
  const int64_t chunks = A.page_bytes / 16;
  const unsigned bx = (unsigned)std::min<int64_t>(64, (chunks + 255) / 256);
  hipLaunchKernelGGL(page_copy_kernel, dim3(bx, (unsigned)A.n_pairs), dim3(256), 0, st, A);
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

}  // namespace pa
