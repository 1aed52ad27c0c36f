"""GPU parity at the five full workload sizes, in the launch shapes bench.py
times.  The oracle checks every output row where it finishes in seconds and
a sample of rows elsewhere; byte-identity rules are checked on whole
outputs."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import paged_kv_cache_addressing_amd as pa
import workloads
from paged_kv_cache_addressing_amd.resident import upload
from tests._gpu import decode, launch_error, prefill, references, same_bytes, say, tol

pytestmark = pytest.mark.gpu

THREADS = 16


def test_config1_decode():
    wl = workloads.config1()
    out = decode(upload(wl))
    refs, sels = references(wl, n_threads=THREADS)
    err = launch_error(wl, out, refs, sels)
    say(f"config1: {err:.3e}")
    assert err <= 1e-2


def test_config2_decode_all_rows_and_halves():
    wl = workloads.config2()
    say("config2: upload")
    res = upload(wl)
    out = decode(res)
    # partials + merge as two calls give the same bytes as paged_attn_decode
    ws = pa.decode_workspace(res.cache, res.streams, wl.n_q_heads, wl.split_keys)
    pa.paged_attn_decode_partials(res.cache, res.streams, res.q, ws, sm_scale=res.sm_scale)
    out2 = torch.empty_like(out)
    pa.paged_attn_decode_merge(res.cache, res.streams, out2, ws)
    torch.cuda.synchronize()
    assert same_bytes(out, out2)
    say("config2: oracle")
    refs, sels = references(wl, n_threads=THREADS)
    err = launch_error(wl, out, refs, sels)
    say(f"config2: {err:.3e}")
    assert err <= 1e-2


def test_config3_decode_fp8_mixed_batch_invariance():
    wl = workloads.config3()
    say("config3: upload")
    res = upload(wl)
    out = decode(res)
    say("config3: oracle")
    refs, sels = references(wl, n_threads=THREADS)
    err = launch_error(wl, out, refs, sels)
    say(f"config3: {err:.3e}")
    assert err <= 3e-2
    # every stream alone gives the same bytes as in the mixed paged/slab batch
    for st in res.streams:
        alone = torch.zeros_like(res.q)
        pa.paged_attn_decode(res.cache, [st], res.q, out=alone, sm_scale=res.sm_scale)
        torch.cuda.synchronize()
        r0, r1 = st.row_offset, st.row_offset + st.n_rows
        assert same_bytes(alone[r0:r1], out[r0:r1])
    # paged streams 0-3 also stored as slabs: same bytes
    ks_all = []
    for s in range(4):
        st = res.streams[s]
        ks, vs = pa.alloc_slab(65536, wl.n_kv_heads, wl.head_dim, "fp8")
        store = pa.Stream(65536, 65536, 0, 0, k_slab=ks, v_slab=vs, slab_cap=65536,
                          layout=pa.PA_LAYOUT_SLAB)
        pa.write_kv(res.cache, [store], wl.k_rows[s].cuda(), wl.v_rows[s].cuda())
        ks_all.append(pa.Stream(st.ctx_len, st.n_rows, st.row_offset, st.first_pos, k_slab=ks,
                                v_slab=vs, slab_cap=65536, layout=pa.PA_LAYOUT_SLAB))
    slab_out = decode(res, streams=ks_all + res.streams[4:])
    assert same_bytes(slab_out, out)


def test_config4_prefill_sampled_rows_and_slices():
    wl = workloads.config4()
    say("config4: upload")
    res = upload(wl)
    out = prefill(res)
    st = res.streams[0]
    # 32 slices of 128 rows give the same bytes as one launch
    sliced = torch.zeros_like(out)
    for i in range(32):
        s = pa.Stream(st.ctx_len, 128, 128 * i, st.first_pos + 128 * i, page_table=st.page_table)
        pa.paged_attn_prefill(res.cache, [s], res.q, out=sliced, sm_scale=res.sm_scale)
    torch.cuda.synchronize()
    assert same_bytes(sliced, out)
    # every 31st row (each residue of the row-tile index over the run) plus
    # the tile and slice boundaries
    rows = sorted(set(list(range(0, 4096, 31)) + [127, 128, 129, 2047, 2048, 4095]))
    say(f"config4: oracle on {len(rows)} rows")
    refs, sels = references(wl, rows_per_stream=lambda s, st: rows, n_threads=THREADS)
    err = launch_error(wl, out, refs, sels)
    say(f"config4: {err:.3e}")
    assert err <= 1e-2


def test_config5_verify_sampled_rows_decode_and_prefill_paths():
    wl = workloads.config5()
    say("config5: upload")
    res = upload(wl)
    out = decode(res)
    out_pf = prefill(res)
    # stream s checks rows s mod 16, (s + 5) mod 16 and 15: over the batch every
    # row index (hence every MFMA column of the split-mode tile) is compared
    def pick(s, st):
        return sorted({s % 16, (s + 5) % 16, 15})
    say("config5: oracle")
    refs, sels = references(wl, rows_per_stream=pick, n_threads=THREADS)
    err = launch_error(wl, out, refs, sels)
    err_pf = launch_error(wl, out_pf, refs, sels)
    say(f"config5: decode {err:.3e}, prefill path {err_pf:.3e}")
    assert err <= 3e-2 and err_pf <= 3e-2
    for _ in range(3):
        assert same_bytes(decode(res), out)
