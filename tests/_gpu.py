"""GPU-test helpers: run the HIP path through the C ABI and compare it with
the oracle.  The expected values always come from ``oracle`` on the host."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
import paged_kv_cache_addressing_amd as pa
from paged_kv_cache_addressing_amd.resident import upload
from tests._util import oracle_pool, oracle_reference

BF16_TOL = 1e-2
FP8_TOL = 3e-2


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def tol(wl) -> float:
    return BF16_TOL if wl.kv_dtype == "bf16" else FP8_TOL


def decode(res, streams=None, q=None, split_keys=None):
    out = pa.paged_attn_decode(res.cache, streams or res.streams, res.q if q is None else q,
                               sm_scale=res.sm_scale, split_keys=split_keys or res.split_keys)
    torch.cuda.synchronize()
    return out


def prefill(res, streams=None, q=None, out=None):
    out = pa.paged_attn_prefill(res.cache, streams or res.streams, res.q if q is None else q,
                                out=out, sm_scale=res.sm_scale)
    torch.cuda.synchronize()
    return out


def references(wl, rows_per_stream=None, n_threads=0):
    """Oracle outputs per stream ([n_sel][Hq][D] float64) and the row indices used."""
    pool = None
    if any(st.layout == "paged" for st in wl.streams):
        pool = oracle_pool(wl)
    refs, sels = [], []
    for s, st in enumerate(wl.streams):
        sel = None if rows_per_stream is None else rows_per_stream(s, st)
        r = oracle_reference(wl, s, rows=sel, pool=pool, n_threads=n_threads)
        refs.append(r)
        sels.append(np.arange(st.n_rows) if sel is None else np.asarray(sel))
    return refs, sels


def launch_error(wl, out, refs, sels):
    """max|gpu - ref| / max|ref| over every compared output of the launch."""
    o = out.float().cpu().numpy()
    got, want = [], []
    for st, ref, sel in zip(wl.streams, refs, sels):
        got.append(o[st.row_offset + sel])
        want.append(ref)
    got = np.concatenate(got)
    want = np.concatenate(want)
    assert np.isfinite(got).all(), "non-finite output"
    return oracle.normalised_error(got, want)


def same_bytes(a: torch.Tensor, b: torch.Tensor) -> bool:
    return torch.equal(a.view(torch.int16), b.view(torch.int16))
