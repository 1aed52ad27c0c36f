"""GPU tests of calls wider than one launch group and of slices that cross
streams, through the C ABI.

A launch carries at most 32 stream descriptors in its kernel arguments, so
larger calls are cut into several launch groups (decode partials and merge,
prefill and write_kv alike), each with group-relative row numbering and
global workspace slots.  The pages' slice test runs two-stream batches where
some slices cross from one stream into the next (TensorFold pull request
#1355, follow-up checks, "Row counts"); here every slicing must give the
bytes of one launch.  Expected values come from the float64 oracle."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import paged_kv_cache_addressing_amd as pa
import workloads
from paged_kv_cache_addressing_amd.resident import upload
from tests._gpu import decode, launch_error, prefill, references, same_bytes, say, tol
from tests._util import gpu_v_layout, oracle_pool

pytestmark = pytest.mark.gpu


def _mixed_batch(dtype, n_streams, seed):
    """Narrow (1-3 rows) and wide (16 rows) decode streams, paged and slab,
    every third wide stream with a random draft tree."""
    rng = np.random.default_rng(seed)
    lens = [int(x) for x in rng.integers(300, 3500, n_streams)]
    rows = [[1, 3, 16][i % 3] for i in range(n_streams)]
    layouts = ["slab" if i % 4 == 1 else "paged" for i in range(n_streams)]
    trees = ["random" if (rows[i] == 16 and i % 2 == 0) else None for i in range(n_streams)]
    return workloads.build(f"batch{n_streams}-{dtype}", n_q_heads=12, n_kv_heads=2, head_dim=128,
                           kv_dtype=dtype, ctx_lens=lens, n_rows=rows, layouts=layouts,
                           seed=seed, split_keys=1024, trees=trees)


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_decode_beyond_one_launch_group_matches_oracle_and_alone(dtype):
    wl = _mixed_batch(dtype, 41, 201)
    res = upload(wl, poison_tail=True)
    _, plan = pa.paged_attn_decode_plan(res.streams, 12, 2, 128, 1024, dtype)
    assert plan.n_launch_groups == 2
    say(f"decode 41 streams {dtype}")
    out = decode(res)
    refs, sels = references(wl)
    err = launch_error(wl, out, refs, sels)
    say(f"decode 41 streams {dtype}: normalised error {err:.3e}")
    assert err <= tol(wl)
    for i, st in enumerate(res.streams):
        alone = torch.zeros_like(res.q)
        pa.paged_attn_decode(res.cache, [st], res.q, out=alone, sm_scale=res.sm_scale,
                             split_keys=1024)
        torch.cuda.synchronize()
        r0, r1 = st.row_offset, st.row_offset + st.n_rows
        assert same_bytes(alone[r0:r1], out[r0:r1]), f"stream {i} alone differs"


def test_prefill_and_store_beyond_one_launch_group():
    rng = np.random.default_rng(202)
    n = 36
    lens = [int(x) for x in rng.integers(200, 1200, n)]
    rows = [int(min(L, r)) for L, r in zip(lens, rng.integers(1, 140, n))]
    layouts = ["slab" if i % 5 == 2 else "paged" for i in range(n)]
    wl = workloads.build("pf36", n_q_heads=6, n_kv_heads=2, head_dim=256, kv_dtype="bf16",
                         ctx_lens=lens, n_rows=rows, layouts=layouts, seed=202)
    say("store 36 streams")
    res = upload(wl)  # one write_kv call storing all 36 streams (two launch groups)
    kp, vp = oracle_pool(wl)
    assert np.array_equal(res.cache.k_pages.cpu().view(torch.int16).numpy().view(np.uint16), kp)
    assert np.array_equal(res.cache.v_pages.cpu().view(torch.int16).numpy().view(np.uint16),
                          gpu_v_layout(vp, pa.v_block("bf16")))
    say("prefill 36 streams")
    out = prefill(res)
    refs, sels = references(wl)
    err = launch_error(wl, out, refs, sels)
    say(f"prefill 36 streams: normalised error {err:.3e}")
    assert err <= tol(wl)
    for st in (res.streams[0], res.streams[33], res.streams[35]):
        alone = torch.zeros_like(res.q)
        pa.paged_attn_prefill(res.cache, [st], res.q, out=alone, sm_scale=res.sm_scale)
        torch.cuda.synchronize()
        r0, r1 = st.row_offset, st.row_offset + st.n_rows
        assert same_bytes(alone[r0:r1], out[r0:r1])


def _cut(st, a, b):
    """Rows [a, b) of stream descriptor st as a descriptor of their own."""
    return pa.Stream(st.ctx_len, b - a, st.row_offset + a, st.first_pos + a,
                     page_table=st.page_table, k_slab=st.k_slab, v_slab=st.v_slab,
                     slab_cap=st.slab_cap, layout=st.layout, tree_mask=None)


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_prefill_slices_crossing_streams_equal_one_launch(dtype):
    """Two streams' rows, 300 and 200, cut into calls of 127, 129 and 244
    rows: the second call holds the end of stream A and the start of stream
    B, the third the rest of B."""
    wl = workloads.build("cross", n_q_heads=6, n_kv_heads=2, head_dim=256, kv_dtype=dtype,
                         ctx_lens=[900, 700], n_rows=[300, 200], layouts=["paged", "slab"],
                         seed=203)
    res = upload(wl)
    one = prefill(res)
    A, B = res.streams
    for calls in ([[(A, 0, 127)], [(A, 127, 256)], [(A, 256, 300), (B, 0, 85)],
                   [(B, 85, 200)]],
                  [[(A, 0, 1)], [(A, 1, 300), (B, 0, 1)], [(B, 1, 200)]],
                  [[(B, 0, 100), (A, 200, 300)], [(A, 0, 200), (B, 100, 200)]]):
        out = torch.zeros_like(res.q)
        for call in calls:
            pa.paged_attn_prefill(res.cache, [_cut(st, a, b) for st, a, b in call], res.q,
                                  out=out, sm_scale=res.sm_scale)
        torch.cuda.synchronize()
        assert same_bytes(out, one), f"slices {[[(a, b) for _, a, b in c] for c in calls]}"
    refs, sels = references(wl)
    assert launch_error(wl, one, refs, sels) <= tol(wl)


def test_decode_on_a_side_stream_keeps_its_workspace():
    """A call on another HIP stream with no workspace given: the workspace the
    binding allocates on torch's current stream must not be handed out again
    while the side stream's kernels still use it."""
    wl = workloads.build("side", n_q_heads=24, n_kv_heads=4, head_dim=256, kv_dtype="fp8",
                         ctx_lens=[60000, 30000], n_rows=[16, 1], seed=204)
    res = upload(wl)
    want = decode(res)
    nb = pa.paged_attn_decode_workspace_size(res.streams, 24, 256)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    out = torch.zeros_like(res.q)
    pa.paged_attn_decode(res.cache, res.streams, res.q, out=out, sm_scale=res.sm_scale,
                         stream=side)
    # fresh allocations on the current stream while the side stream runs: had
    # the workspace block been released, these fills would land in it
    junk = [torch.full((nb,), 0x7F, dtype=torch.uint8, device="cuda") for _ in range(4)]
    torch.cuda.synchronize()
    del junk
    assert same_bytes(out, want)
