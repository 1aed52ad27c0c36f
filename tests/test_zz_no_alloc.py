"""paged_attn_decode_noalloc, through the C ABI, against paged_attn_decode.

The no-allocation entry point keeps the split partials in the library's
fixed device scratch instead of a caller workspace; it runs the same kernels,
so its output bytes must equal paged_attn_decode's.  Two calls in a row, the
second on a smaller input, check that the scratch's leftover contents from
the first call never reach the second; a call whose partials exceed the
scratch is refused before anything launches."""
from __future__ import annotations

import pytest
import torch

import paged_kv_cache_addressing_amd as pa
import workloads
from paged_kv_cache_addressing_amd.resident import upload
from tests._gpu import decode, launch_error, references, same_bytes, say, tol

pytestmark = pytest.mark.gpu


def _noalloc(res, streams=None):
    out = torch.full_like(res.q, float("nan"))
    pa.paged_attn_decode_noalloc(res.cache, streams or res.streams, res.q, out,
                                 sm_scale=res.sm_scale, split_keys=res.split_keys)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_noalloc_decode_equals_workspace_decode_twice(dtype):
    big = workloads.build("noalloc-big", n_q_heads=24, n_kv_heads=4, head_dim=256,
                          kv_dtype=dtype, ctx_lens=[20000, 9000, 4097, 700],
                          n_rows=[16, 1, 16, 3], seed=101)
    small = workloads.build("noalloc-small", n_q_heads=24, n_kv_heads=4, head_dim=256,
                            kv_dtype=dtype, ctx_lens=[5000, 300], n_rows=[2, 16], seed=102)
    for wl in (big, small):
        say(f"noalloc {dtype} {wl.name}")
        res = upload(wl, poison_tail=True)
        want = decode(res)
        got = _noalloc(res)
        assert same_bytes(got, want), f"{wl.name}: noalloc bytes differ from the workspace call"
        refs, sels = references(wl)
        err = launch_error(wl, got, refs, sels)
        say(f"noalloc {dtype} {wl.name}: normalised error {err:.3e}")
        assert err <= tol(wl)


def test_noalloc_refuses_partials_beyond_the_scratch():
    # 16 streams x 16 rows x 24 heads at 1,024-key splits over 32,768 keys:
    # 16*16*24*32 = 196,608 partials of 1 KiB, more than the scratch holds
    streams = [pa.Stream(32768, 16, 16 * i, 32768 - 16, page_table=torch.zeros(
        128, dtype=torch.int32, device="cuda")) for i in range(16)]
    cache = pa.alloc_pool(1, 4, 256, "bf16")
    assert pa.paged_attn_decode_workspace_size(streams, 24, 256, 1024) > pa.NOALLOC_SCRATCH_BYTES
    q = torch.zeros((256, 24, 256), dtype=torch.bfloat16, device="cuda")
    out = torch.zeros_like(q)
    with pytest.raises(pa.PagedAttnError) as e:
        pa.paged_attn_decode_noalloc(cache, streams, q, out, split_keys=1024)
    assert e.value.status == pa.PA_EWORKSPACE
    torch.cuda.synchronize()
    assert bool((out == 0).all())  # nothing was launched
