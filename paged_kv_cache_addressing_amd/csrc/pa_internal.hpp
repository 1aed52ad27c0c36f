// Launchers shared between the kernel translation units and the C ABI layer.
// Each returns 0, -6 (launch failed) or -7 (no kernel for the shape).
#pragma once

#include <hip/hip_runtime.h>

#include <algorithm>

#include "pa_kargs.hpp"

namespace pa {

int launch_decode_partials(const DecodeArgs& A, int kv_dtype, int head_dim, int n_kv_heads,
                           hipStream_t st);
int launch_decode_merge(const DecodeArgs& A, int head_dim, hipStream_t st);
// MFMA columns ((row, q head) pairs) one column group of the row-tile
// kernel covers (a wave, or a producer/consumer wave pair), in prefill or
// in split mode.
int prefill_columns(int kv_dtype, int head_dim, bool split);
// MFMA columns one row-tile workgroup covers (all its column groups).
int prefill_wg_columns(int kv_dtype, int head_dim, bool split);
int launch_prefill(const PrefillArgs& A, int kv_dtype, int head_dim, hipStream_t st);
// fp8 verify kernel: split-K partials of decode streams with many columns
// (PrefillArgs in split mode, fp8 KV).
int verify_wg_columns(int head_dim);
int launch_verify(const PrefillArgs& A, int head_dim, hipStream_t st);
int launch_write_kv(const WriteArgs& A, int kv_dtype, int head_dim, hipStream_t st);
int launch_page_copy(const PageCopyArgs& A, hipStream_t st);
// Streaming read of bytes (a positive multiple of 16) at buf (16-byte
// aligned), folded into *sink.
int launch_hbm_read_probe(const void* buf, int64_t bytes, uint32_t* sink, hipStream_t st);

// Bytes of the fixed device scratch behind paged_attn_decode_noalloc.
constexpr size_t kNoAllocScratchBytes = (size_t)128 << 20;
// Device address of the current device's scratch (looked up once per
// device); returns 0, or -6 if the lookup failed.
int noalloc_scratch(void** ptr);

}  // namespace pa
