// Plain streaming read of a device buffer: the reference rate against which
// the attention kernels' HBM fractions are read (the timing method of the
// pages' A/A and ABBA measurements interleaves such a probe with the timed
// arms).  The buffer is cut into one contiguous run per workgroup, read in
// 32 KiB steps (each wave 4 x 1 KiB per step) with four steps of nontemporal
// register loads in flight, the access shape that reads fastest on this
// device.  Every 16-byte chunk is read once and folded into one word per
// workgroup, so that no load is dead; the folded words are XORed into *sink.
#include "pa_device.hpp"
#include "pa_internal.hpp"

namespace pa {

namespace {
constexpr int kProbeBlocks = 1024;
constexpr int kProbeThreads = 512;
constexpr int kProbeStep = 2048;  // 16-byte chunks per workgroup step (32 KiB)
constexpr int kProbeLead = 4;     // steps in flight
}  // namespace

__global__ __launch_bounds__(kProbeThreads) void hbm_read_probe_kernel(const v4u* __restrict__ p,
                                                                      int64_t n16,
                                                                      uint32_t* sink) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t per_wg = n16 / kProbeBlocks;
  const v4u* base = p + (int64_t)blockIdx.x * per_wg;
  const int64_t steps = per_wg / kProbeStep;
  uint32_t acc = 0;
  v4u r[kProbeLead][4];
  auto ld = [&](int64_t st, v4u (&x)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      x[i] = __builtin_nontemporal_load(base + st * kProbeStep + (wave * 4 + i) * 64 + lane);
  };
#pragma unroll
  for (int j = 0; j < kProbeLead; ++j)
    if (j < steps) ld(j, r[j]);
  for (int64_t st = 0; st < steps; st += kProbeLead) {
#pragma unroll
    for (int j = 0; j < kProbeLead; ++j) {
      if (st + j < steps) {
#pragma unroll
        for (int i = 0; i < 4; ++i) acc ^= r[j][i][0] ^ r[j][i][1] ^ r[j][i][2] ^ r[j][i][3];
        if (st + j + kProbeLead < steps) ld(st + j + kProbeLead, r[j]);
      }
    }
  }
  // the workgroup's chunks past its whole steps, then (workgroup 0) the
  // chunks past the last workgroup's run
  for (int64_t c = steps * kProbeStep + tid; c < per_wg; c += kProbeThreads) {
    const v4u x = __builtin_nontemporal_load(base + c);
    acc ^= x[0] ^ x[1] ^ x[2] ^ x[3];
  }
  if (blockIdx.x == 0)
    for (int64_t c = per_wg * kProbeBlocks + tid; c < n16; c += kProbeThreads) {
      const v4u x = __builtin_nontemporal_load(p + c);
      acc ^= x[0] ^ x[1] ^ x[2] ^ x[3];
    }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, off, 64);
  // one atomic per workgroup: the waves' words meet in LDS first
  __shared__ uint32_t fold[kProbeThreads / 64];
  if (lane == 0) fold[wave] = acc;
  __syncthreads();
  if (tid == 0) {
    uint32_t f = 0;
#pragma unroll
    for (int w = 0; w < kProbeThreads / 64; ++w) f ^= fold[w];
    atomicXor(sink, f);
  }
}

int launch_hbm_read_probe(const void* buf, int64_t bytes, uint32_t* sink, hipStream_t st) {
  hipLaunchKernelGGL(hbm_read_probe_kernel, dim3(kProbeBlocks), dim3(kProbeThreads), 0, st,
                     static_cast<const v4u*>(buf), bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

}  // namespace pa
