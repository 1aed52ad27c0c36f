"""GPU parity at small sizes (several tiles, ragged tails, edge cases) and the
byte-identity rules, through the C ABI.  Expected values come from the
float64 oracle; byte-identity checks compare the HIP path with itself."""
from __future__ import annotations

import copy

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_addressing_amd as pa
import workloads
from paged_kv_cache_addressing_amd.resident import upload
from tests._gpu import decode, launch_error, prefill, references, same_bytes, say, tol
from tests._util import bits16, gpu_v_layout, oracle_logical, oracle_pool

pytestmark = pytest.mark.gpu


def as_slabs(wl):
    """The same workload with every stream stored in a slab."""
    w = copy.copy(wl)
    w.streams = []
    for st in wl.streams:
        s = copy.copy(st)
        s.layout = "slab"
        s.pages = None
        s.slab_cap = -(-st.ctx_len // 256) * 256
        w.streams.append(s)
    return w


def np_bits(t: torch.Tensor) -> np.ndarray:
    t = t.cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


# ----------------------------------------------------------------------------- write_kv

@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
@pytest.mark.parametrize("d", [128, 256])
def test_write_kv_bytes_match_oracle_store(dtype, d):
    wl = workloads.build("store", n_q_heads=4, n_kv_heads=2, head_dim=d, kv_dtype=dtype,
                         ctx_lens=[700, 300, 513], n_rows=[1, 1, 1],
                         layouts=["paged", "slab", "paged"], n_pages=8, seed=5)
    say(f"write_kv {dtype} D={d}")
    res = upload(wl)
    vb = pa.v_block(dtype)
    kp, vp = oracle_pool(wl)  # [pages][Hkv][256][D], the pages' head-major layout
    assert np.array_equal(np_bits(res.cache.k_pages), kp)
    assert np.array_equal(np_bits(res.cache.v_pages), gpu_v_layout(vp, vb))
    k_log, v_log = oracle_logical(wl, 1)  # [300][Hkv][D]
    ks, vs = res.slabs[1]
    cap = ks.shape[1]
    k_full = np.zeros((2, cap, d), k_log.dtype)
    v_full = np.zeros((2, cap, d), v_log.dtype)
    k_full[:, :300] = k_log.transpose(1, 0, 2)
    v_full[:, :300] = v_log.transpose(1, 0, 2)
    assert np.array_equal(np_bits(ks), k_full)
    assert np.array_equal(np_bits(vs), gpu_v_layout(v_full, vb))


@pytest.mark.parametrize("scale", [1.0, 0.0107421875, 3.7])
def test_fp8_store_every_finite_bf16_value(scale):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = oracle.bf16_to_f64(bits)
    fin = bits[np.isfinite(vals)]
    assert fin.size == 65280
    rows = torch.from_numpy(fin.view(np.int16).copy()).view(torch.bfloat16).reshape(510, 1, 128)
    cache = pa.alloc_pool(1, 1, 128, "fp8")
    cache.k_scale, cache.v_scale = scale, scale * 2
    ks, vs = pa.alloc_slab(512, 1, 128, "fp8")
    st = pa.Stream(510, 510, 0, 0, k_slab=ks, v_slab=vs, slab_cap=512, layout=pa.PA_LAYOUT_SLAB)
    dev = rows.cuda()
    pa.write_kv(cache, [st], dev, dev)
    torch.cuda.synchronize()
    x32 = oracle.bf16_to_f64(fin).astype(np.float32)
    want_k = oracle.e4m3_encode(x32, scale).reshape(510, 128)
    want_v = oracle.e4m3_encode(x32, scale * 2).reshape(510, 128)
    got_k = ks.cpu().numpy()[0, :510, :]
    got_v = np.swapaxes(vs.cpu().numpy()[0], -1, -2).reshape(512, 128)[:510]
    bad = np.nonzero(got_k != want_k)
    assert bad[0].size == 0, (x32.reshape(510, 128)[bad][:8], got_k[bad][:8], want_k[bad][:8])
    assert np.array_equal(got_v, want_v)


# ----------------------------------------------------------------------------- decode

DECODE_CASES = [
    # name, Hq, Hkv, D, dtype, ctx_lens, rows, layouts, split
    ("c1", 8, 2, 128, "bf16", [1024], [1], None, 4096),
    ("ragged-bf16", 24, 4, 256, "bf16", [5000, 300, 4097, 1], [1, 1, 1, 1], None, 4096),
    ("ragged-fp8-mixed", 24, 4, 256, "fp8", [5000, 9000, 257], [1, 1, 1],
     ["paged", "slab", "paged"], 4096),
    ("verify-bf16-d128", 12, 2, 128, "bf16", [2000, 4103], [16, 3], None, 1024),
    ("verify-fp8-masked-split", 24, 4, 256, "fp8", [4100, 6000, 4096 + 16], [16, 16, 16],
     None, 4096),
    ("small-split", 6, 1, 256, "bf16", [3000], [5], None, 256),
    # more than 256 splits per row (the merge stages split weights 256 at a
    # time) and one-page splits (the page walk's rotation is the identity)
    ("many-splits", 8, 2, 128, "bf16", [70000, 600], [1, 2], ["paged", "slab"], 256),
    # verify rows on the LDS-shared row-tile kernel in split mode
    ("verify-bf16-d256-mixed", 24, 4, 256, "bf16", [3 * 4096 + 5, 9000, 316], [16, 16, 16],
     ["paged", "slab", "paged"], 4096),
    ("verify-g16-d128-two-tiles", 32, 2, 128, "bf16", [5000], [16], None, 2048),
    ("verify-g8-d256-fp8", 32, 4, 256, "fp8", [9000, 4096], [16, 9], None, 4096),
    # bf16 at head_dim 256 runs producer/consumer wave pairs: 8 heads per tile
    ("verify-g8-d256-bf16", 32, 4, 256, "bf16", [9000, 4096], [16, 9], None, 4096),
    # register-streaming kernel with two column tiles (3 rows x 8 heads) and
    # with one q head per kv head
    ("narrow-g8-d256", 32, 4, 256, "bf16", [7000, 300], [3, 2], None, 4096),
    ("mha-d256-fp8", 4, 4, 256, "fp8", [3000, 8193], [2, 1], ["slab", "paged"], 4096),
    # every stream one split: the partial kernel writes the rows itself (no
    # merge), at head_dim 256 for both KV dtypes
    ("one-split-d256-bf16", 24, 4, 256, "bf16", [300, 4096, 1], [3, 1, 1], None, 4096),
    ("one-split-d256-fp8", 24, 4, 256, "fp8", [4096, 2500, 2], [1, 2, 1],
     ["paged", "slab", "paged"], 4096),
]


@pytest.mark.parametrize("case", DECODE_CASES, ids=[c[0] for c in DECODE_CASES])
def test_decode_matches_oracle(case):
    name, hq, hkv, d, dtype, lens, rows, layouts, split = case
    wl = workloads.build(name, n_q_heads=hq, n_kv_heads=hkv, head_dim=d, kv_dtype=dtype,
                         ctx_lens=lens, n_rows=rows, layouts=layouts, seed=11,
                         split_keys=split)
    say(f"decode {name}")
    res = upload(wl, poison_tail=True)
    out = decode(res)
    refs, sels = references(wl)
    err = launch_error(wl, out, refs, sels)
    say(f"decode {name}: normalised error {err:.3e}")
    assert err <= tol(wl)


def test_decode_config1_exact_shape():
    wl = workloads.config1()
    res = upload(wl)
    out = decode(res)
    refs, sels = references(wl)
    err = launch_error(wl, out, refs, sels)
    say(f"decode config1: {err:.3e}")
    assert err <= 1e-2


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_decode_byte_identities(dtype):
    """paged == slab, alone == beside others, five repeats: all byte-equal."""
    wl = workloads.build("ident", n_q_heads=24, n_kv_heads=4, head_dim=256, kv_dtype=dtype,
                         ctx_lens=[9000, 4097, 700], n_rows=[1, 16, 3], seed=21)
    res = upload(wl)
    base = decode(res)
    for _ in range(5):
        assert same_bytes(decode(res), base)
    slab = upload(as_slabs(wl))
    assert same_bytes(decode(slab), base)
    for i, st in enumerate(res.streams):
        out = torch.zeros_like(res.q)
        pa.paged_attn_decode(res.cache, [st], res.q, out=out, sm_scale=res.sm_scale)
        torch.cuda.synchronize()
        r0, r1 = st.row_offset, st.row_offset + st.n_rows
        assert same_bytes(out[r0:r1], base[r0:r1]), f"stream {i} alone differs"
    # beside a slab stream in the same launch
    mixed = [res.streams[0], slab.streams[1], res.streams[2]]
    assert same_bytes(decode(res, streams=mixed), base)


def test_decode_swapped_table_control_fails():
    wl = workloads.build("swap", n_q_heads=8, n_kv_heads=2, head_dim=128, kv_dtype="bf16",
                         ctx_lens=[1024], n_rows=[1], n_pages=8, seed=1001)
    res = upload(wl)
    good = decode(res)
    refs, sels = references(wl)
    assert launch_error(wl, good, refs, sels) <= 1e-2
    pt = res.page_tables[0]
    bad = pt.clone()
    bad[1] = int(wl.filler_pages[0])  # an unused pool page instead of the stream's own
    st = pa.Stream(1024, 1, 0, 1023, page_table=bad)
    out = decode(res, streams=[st])
    assert not same_bytes(out, good)
    assert launch_error(wl, out, refs, sels) > 1e-2


def test_decode_poisoned_tail_is_never_read():
    wl = workloads.build("poison", n_q_heads=24, n_kv_heads=4, head_dim=256, kv_dtype="fp8",
                         ctx_lens=[1000, 257], n_rows=[1, 2], seed=31)
    clean = decode(upload(wl))
    poisoned = decode(upload(wl, poison_tail=True))
    assert torch.isfinite(poisoned.float()).all()
    assert same_bytes(clean, poisoned)


def _with_table(st, table):
    return pa.Stream(st.ctx_len, st.n_rows, st.row_offset, st.first_pos, page_table=table)


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_rejected_page_ids_poison_only_their_stream(dtype):
    """A page id outside [0, n_pages) is never dereferenced: the rows computed
    with it come out NaN, and every other stream keeps its bytes."""
    wl = workloads.build("badid", n_q_heads=24, n_kv_heads=4, head_dim=256, kv_dtype=dtype,
                         ctx_lens=[3000, 5000, 900], n_rows=[1, 16, 3], seed=71)
    res = upload(wl)
    n_pages = res.cache.n_pages
    base_dec = decode(res)
    base_pf = prefill(res)
    t0 = res.page_tables[0].clone()
    t0[5] = n_pages + 3            # past the pool (narrow decode stream)
    t1 = res.page_tables[1].clone()
    t1[-1] = -1                    # negative (verify rows on the row-tile kernel)
    bad = [_with_table(res.streams[0], t0), _with_table(res.streams[1], t1), res.streams[2]]
    out = decode(res, streams=bad)
    for st in res.streams[:2]:
        rows = out[st.row_offset:st.row_offset + st.n_rows].float()
        assert torch.isnan(rows).all(), "a row computed with a rejected page id is not NaN"
    r0, r1 = res.streams[2].row_offset, res.streams[2].row_offset + res.streams[2].n_rows
    assert same_bytes(out[r0:r1], base_dec[r0:r1])
    # prefill: every row reads page 0
    t2 = res.page_tables[2].clone()
    t2[0] = n_pages
    pf = prefill(res, streams=[res.streams[0], res.streams[1], _with_table(res.streams[2], t2)])
    assert torch.isnan(pf[r0:r1].float()).all()
    assert same_bytes(pf[:r0], base_pf[:r0])


def test_write_kv_skips_rows_with_rejected_page_ids():
    wl = workloads.build("badstore", n_q_heads=8, n_kv_heads=2, head_dim=128, kv_dtype="bf16",
                         ctx_lens=[600, 600], n_rows=[1, 1], seed=72)
    res = upload(wl)
    k0, v0 = res.cache.k_pages.clone(), res.cache.v_pages.clone()
    t = res.page_tables[0].clone()
    t[2] = res.cache.n_pages + 1   # position 599 lives in page 2
    rows = torch.randn(2, 2, 128).to(torch.bfloat16).cuda()
    st_bad = pa.Stream(600, 1, 0, 599, page_table=t)
    st_good = pa.Stream(600, 1, 1, 599, page_table=res.page_tables[1])
    pa.write_kv(res.cache, [st_bad, st_good], rows, rows)
    torch.cuda.synchronize()
    changed = (res.cache.k_pages.view(torch.int16) != k0.view(torch.int16))
    pages = sorted(set(torch.nonzero(changed)[:, 0].tolist()))
    assert pages == [int(wl.streams[1].pages[2])], pages  # only the good stream's page
    assert not torch.equal(res.cache.v_pages.view(torch.int16), v0.view(torch.int16))


# ----------------------------------------------------------------------------- prefill

PREFILL_CASES = [
    # name, Hq, Hkv, D, dtype, ctx_lens, rows, layouts
    ("rows1", 6, 2, 256, "bf16", [301], [1], None),
    ("rows127", 6, 2, 256, "bf16", [427], [127], None),
    ("rows128", 6, 2, 256, "bf16", [428], [128], None),
    ("rows129", 6, 2, 256, "bf16", [429], [129], None),
    ("rows257-noprefix", 6, 2, 256, "bf16", [257], [257], None),
    ("d128", 8, 2, 128, "bf16", [900], [300], None),
    ("fp8", 6, 2, 256, "fp8", [1000], [300], None),
    ("two-streams-mixed", 6, 2, 256, "bf16", [700, 1200], [129, 300], ["paged", "slab"]),
    ("fp8-d128-mixed", 4, 1, 128, "fp8", [513, 2000], [200, 77], ["slab", "paged"]),
    # other group sizes on the paired bf16 kernel: 8 heads (16-row tiles) and 1
    ("g8-rows200", 16, 2, 256, "bf16", [1500], [200], None),
    ("g1-mha", 2, 2, 256, "bf16", [600], [130], None),
]


@pytest.mark.parametrize("case", PREFILL_CASES, ids=[c[0] for c in PREFILL_CASES])
def test_prefill_matches_oracle(case):
    name, hq, hkv, d, dtype, lens, rows, layouts = case
    wl = workloads.build(name, n_q_heads=hq, n_kv_heads=hkv, head_dim=d, kv_dtype=dtype,
                         ctx_lens=lens, n_rows=rows, layouts=layouts, seed=41)
    say(f"prefill {name}")
    res = upload(wl, poison_tail=True)
    out = prefill(res)
    refs, sels = references(wl)
    err = launch_error(wl, out, refs, sels)
    say(f"prefill {name}: normalised error {err:.3e}")
    assert err <= tol(wl)


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_prefill_slices_equal_one_launch_and_slab(dtype):
    wl = workloads.build("slices", n_q_heads=6, n_kv_heads=2, head_dim=256, kv_dtype=dtype,
                         ctx_lens=[1600], n_rows=[600], seed=51)
    res = upload(wl)
    one = prefill(res)
    st = res.streams[0]
    for cuts in ([127, 1, 128, 129, 215], [128] * 4 + [88], [257, 256, 87]):
        out = torch.zeros_like(res.q)
        off = 0
        for c in cuts:
            s = pa.Stream(st.ctx_len, c, off, st.first_pos + off, page_table=st.page_table)
            pa.paged_attn_prefill(res.cache, [s], res.q, out=out, sm_scale=res.sm_scale)
            off += c
        torch.cuda.synchronize()
        assert off == 600
        assert same_bytes(out, one), f"slices {cuts} differ from one launch"
    slab = upload(as_slabs(wl))
    assert same_bytes(prefill(slab), one)
    for _ in range(3):
        assert same_bytes(prefill(res), one)


def test_prefill_slices_left_at_row_zero_control_fails():
    wl = workloads.build("slices0", n_q_heads=6, n_kv_heads=2, head_dim=256, kv_dtype="bf16",
                         ctx_lens=[800], n_rows=[256], seed=52)
    res = upload(wl)
    one = prefill(res)
    st = res.streams[0]
    out = torch.zeros_like(res.q)
    for off in (0, 128):
        # planted mistake: the second slice keeps the first slice's position
        s = pa.Stream(st.ctx_len, 128, off, st.first_pos, page_table=st.page_table)
        pa.paged_attn_prefill(res.cache, [s], res.q, out=out, sm_scale=res.sm_scale)
    torch.cuda.synchronize()
    assert not same_bytes(out, one)


def test_prefill_stream_alone_equals_beside_others():
    wl = workloads.build("beside", n_q_heads=6, n_kv_heads=2, head_dim=256, kv_dtype="bf16",
                         ctx_lens=[700, 1200, 300], n_rows=[129, 300, 5],
                         layouts=["paged", "slab", "paged"], seed=53)
    res = upload(wl)
    both = prefill(res)
    for st in res.streams:
        out = torch.zeros_like(res.q)
        pa.paged_attn_prefill(res.cache, [st], res.q, out=out, sm_scale=res.sm_scale)
        torch.cuda.synchronize()
        r0, r1 = st.row_offset, st.row_offset + st.n_rows
        assert same_bytes(out[r0:r1], both[r0:r1])


# ----------------------------------------------------------------------------- partials + merge

@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_decode_partials_match_oracle_split_form(dtype):
    """The workspace triples follow the documented layout and equal the
    oracle's split form (m in log2 units), and merge(partials) == decode."""
    split = 1024
    wl = workloads.build("halves", n_q_heads=12, n_kv_heads=2, head_dim=128, kv_dtype=dtype,
                         ctx_lens=[2500, 1030], n_rows=[3, 16], seed=61, split_keys=split)
    res = upload(wl)
    full = decode(res)
    ws = pa.decode_workspace(res.cache, res.streams, wl.n_q_heads, split)
    ws.fill_(0xFF)  # every byte the merge reads must be written by the partials
    pa.paged_attn_decode_partials(res.cache, res.streams, res.q, ws, sm_scale=res.sm_scale,
                                  split_keys=split)
    out = torch.empty_like(full)
    pa.paged_attn_decode_merge(res.cache, res.streams, out, ws, split_keys=split)
    torch.cuda.synchronize()
    assert same_bytes(out, full)
    kp, vp = oracle_pool(wl)
    ps = wl.n_kv_heads * 256 * wl.head_dim
    d, hq = wl.head_dim, wl.n_q_heads
    slots = sum(st.n_rows * hq * -(-(st.first_pos + st.n_rows) // split) for st in wl.streams)
    wsf = ws.view(torch.float32).cpu().numpy()
    o_all = wsf[:slots * d].reshape(slots, d)
    ml_off = -(-(slots * d * 4) // 256) * 256 // 4
    ml = wsf[ml_off:ml_off + 2 * slots].reshape(slots, 2)
    base = 0
    for st in wl.streams:
        ns = -(-(st.first_pos + st.n_rows) // split)
        q = bits16(wl.q[st.row_offset:st.row_offset + st.n_rows])
        m, l, o = oracle.attention_split(kp, vp, oracle.DTYPE_BF16 if dtype == "bf16" else
                                         oracle.DTYPE_E4M3, q, st.first_pos, wl.n_kv_heads,
                                         st.ctx_len, split, ns, page_table=st.pages,
                                         page_stride=ps, sm_scale=wl.sm_scale,
                                         k_scale=wl.k_scale, v_scale=wl.v_scale)
        n = st.n_rows * hq * ns
        gm = ml[base:base + n, 0].reshape(st.n_rows, hq, ns)
        gl = ml[base:base + n, 1].reshape(st.n_rows, hq, ns)
        go = o_all[base:base + n].reshape(st.n_rows, hq, ns, d)
        masked = np.isneginf(m)
        assert np.array_equal(np.isneginf(gm), masked)
        assert (gl[masked] == 0).all() and (go[masked] == 0).all()
        vis = ~masked
        # m is a reference logit (log2 units) at most 8 below the split's
        # largest; the split's total weight l * 2^m does not depend on it
        mo = m[vis] / np.log(2.0)
        assert (gm[vis] <= mo + 2e-2).all() and (gm[vis] >= mo - 8 - 2e-2).all()
        np.testing.assert_allclose(np.log2(gl[vis]) + gm[vis], np.log2(l[vis]) + mo, rtol=0,
                                   atol=2e-2)
        vs = wl.v_scale if dtype == "fp8" else 1.0  # o is kept in V-code units
        np.testing.assert_allclose(go[vis] / gl[vis][..., None] * vs, o[vis] / l[vis][..., None],
                                   rtol=0, atol=(2e-2 if dtype == "bf16" else 6e-2))
        base += n


# ----------------------------------------------------------------------------- draft-tree rows

TREE_DECODE_CASES = [
    # name, Hq, Hkv, D, dtype, ctx_lens, rows, layouts, split
    ("tree-wide-bf16-mixed", 24, 4, 256, "bf16", [4100, 9000, 700], [16, 16, 7],
     ["paged", "slab", "paged"], 4096),
    ("tree-wide-fp8", 24, 4, 256, "fp8", [6000, 4096 + 10], [16, 12], None, 4096),
    ("tree-narrow-d128", 12, 2, 128, "bf16", [2000, 1030], [3, 5], None, 1024),
    ("tree-wide-d128-fp8", 12, 2, 128, "fp8", [3000], [16], None, 1024),
]


@pytest.mark.parametrize("case", TREE_DECODE_CASES, ids=[c[0] for c in TREE_DECODE_CASES])
def test_tree_decode_matches_oracle(case):
    name, hq, hkv, d, dtype, lens, rows, layouts, split = case
    wl = workloads.build(name, n_q_heads=hq, n_kv_heads=hkv, head_dim=d, kv_dtype=dtype,
                         ctx_lens=lens, n_rows=rows, layouts=layouts, seed=81,
                         split_keys=split, trees=["random"] * len(lens))
    say(f"tree decode {name}")
    res = upload(wl, poison_tail=True)
    out = decode(res)
    refs, sels = references(wl)
    err = launch_error(wl, out, refs, sels)
    say(f"tree decode {name}: normalised error {err:.3e}")
    assert err <= tol(wl)
    # the tree changes the result (the control: the causal rows differ)
    causal = decode(upload(workloads.build(name, n_q_heads=hq, n_kv_heads=hkv, head_dim=d,
                                           kv_dtype=dtype, ctx_lens=lens, n_rows=rows,
                                           layouts=layouts, seed=81, split_keys=split)))
    assert not same_bytes(causal, out)


@pytest.mark.parametrize("dtype,d,rows", [("bf16", 256, 32), ("fp8", 256, 20), ("bf16", 128, 29)])
def test_tree_prefill_matches_oracle(dtype, d, rows):
    wl = workloads.build("tree-prefill", n_q_heads=8 if d == 128 else 6, n_kv_heads=2,
                         head_dim=d, kv_dtype=dtype, ctx_lens=[900, 333], n_rows=[rows, 7],
                         layouts=["paged", "slab"], seed=82, trees=["random", "random"])
    res = upload(wl, poison_tail=True)
    out = prefill(res)
    refs, sels = references(wl)
    err = launch_error(wl, out, refs, sels)
    say(f"tree prefill {dtype} d{d}: normalised error {err:.3e}")
    assert err <= tol(wl)


def test_chain_tree_gives_the_causal_bytes_and_trees_are_batch_invariant():
    kw = dict(n_q_heads=24, n_kv_heads=4, head_dim=256, kv_dtype="bf16",
              ctx_lens=[5000, 4097, 800], n_rows=[16, 3, 16], seed=83)
    plain = upload(workloads.build("chain", **kw))
    chain = upload(workloads.build("chain", trees=["chain"] * 3, **kw))
    assert same_bytes(decode(chain), decode(plain))
    assert same_bytes(prefill(chain), prefill(plain))
    tree = upload(workloads.build("tree", trees=["random", None, "random"], **kw))
    both = decode(tree)
    for st in tree.streams:
        alone = torch.zeros_like(tree.q)
        pa.paged_attn_decode(tree.cache, [st], tree.q, out=alone, sm_scale=tree.sm_scale)
        torch.cuda.synchronize()
        r0, r1 = st.row_offset, st.row_offset + st.n_rows
        assert same_bytes(alone[r0:r1], both[r0:r1])


# ----------------------------------------------------------------------------- guards and controls

def _guarded(n_bytes: int, guard: int = 4096):
    """A uint8 device buffer with `guard` canary bytes (0xA5) on each side of
    an n_bytes window; returns (buffer, window)."""
    buf = torch.full((n_bytes + 2 * guard,), 0xA5, dtype=torch.uint8, device="cuda")
    return buf, buf[guard:guard + n_bytes]


def _guards_intact(buf: torch.Tensor, n_bytes: int, guard: int = 4096) -> bool:
    return bool((buf[:guard] == 0xA5).all()) and bool((buf[guard + n_bytes:] == 0xA5).all())


@pytest.mark.parametrize("n_streams,spw", [(8, 2), (10, 3)])
def test_decode_split_groups_equal_alone_and_stay_in_their_buffers(n_streams, spw):
    """8 (10) streams of 16 splits make 512 (640) one-split workgroups, more
    than two rounds, so each workgroup computes 2 (3) consecutive 1,024-key
    splits (with 3, each stream's last workgroup has one split); every stream
    alone (64 workgroups, one split each) gives the same bytes.  Workspace and
    output sit between canary bytes that must survive."""
    wl = workloads.build("groups", n_q_heads=24, n_kv_heads=4, head_dim=256, kv_dtype="bf16",
                         ctx_lens=[16384] * n_streams, n_rows=[1] * n_streams, split_keys=1024,
                         seed=91)
    res = upload(wl)
    _, plan = pa.paged_attn_decode_plan(res.streams, 24, 4, 256, 1024)
    assert plan.narrow_splits_per_wg == spw
    nb = pa.paged_attn_decode_workspace_size(res.streams, 24, 256, 1024)
    wbuf, ws = _guarded(nb)
    ob = res.q.numel() * 2
    obuf, ow = _guarded(ob)
    out = ow.view(torch.bfloat16).view(res.q.shape)
    pa.paged_attn_decode(res.cache, res.streams, res.q, out=out, sm_scale=res.sm_scale,
                         split_keys=1024, workspace=ws)
    torch.cuda.synchronize()
    assert _guards_intact(wbuf, nb) and _guards_intact(obuf, ob)
    refs, sels = references(wl)
    err = launch_error(wl, out, refs, sels)
    say(f"split groups: normalised error {err:.3e}")
    assert err <= tol(wl)
    for st in res.streams:
        alone = decode(res, streams=[st], split_keys=1024)
        r0, r1 = st.row_offset, st.row_offset + st.n_rows
        assert same_bytes(alone[r0:r1], out[r0:r1])


def test_prefill_output_stays_in_its_buffer():
    wl = workloads.build("pf-guard", n_q_heads=24, n_kv_heads=4, head_dim=256, kv_dtype="bf16",
                         ctx_lens=[700, 1500], n_rows=[300, 77], seed=92)
    res = upload(wl)
    ob = res.q.numel() * 2
    obuf, ow = _guarded(ob)
    out = ow.view(torch.bfloat16).view(res.q.shape)
    prefill(res, out=out)
    assert _guards_intact(obuf, ob)
    assert same_bytes(out, prefill(res))


def test_fp8_swapped_scales_control_fails():
    """V carries 8 times K's scale (V rows times 8 store the same codes); the
    launch matches the oracle with the right scales and not with K's and V's
    scales swapped."""
    wl = workloads.build("scales", n_q_heads=24, n_kv_heads=4, head_dim=256, kv_dtype="fp8",
                         ctx_lens=[3000, 5000], n_rows=[1, 16], seed=93)
    wl.v_rows = [(v.float() * 8).to(torch.bfloat16) for v in wl.v_rows]
    wl.v_scale = wl.v_scale * 8
    res = upload(wl)
    refs, sels = references(wl)
    err = launch_error(wl, decode(res), refs, sels)
    assert err <= tol(wl)
    res.cache.k_scale, res.cache.v_scale = res.cache.v_scale, res.cache.k_scale
    bad = launch_error(wl, decode(res), refs, sels)
    say(f"scales: {err:.3e} right, {bad:.3e} swapped")
    assert bad > tol(wl)


def test_context_past_the_stored_rows_control_reads_poison():
    """A descriptor that claims one position more than was stored makes its
    row read the poisoned slot after the stream's last key: NaN."""
    wl = workloads.build("ctx+1", n_q_heads=24, n_kv_heads=4, head_dim=256, kv_dtype="bf16",
                         ctx_lens=[3000], n_rows=[1], seed=94)
    res = upload(wl, poison_tail=True)
    st = res.streams[0]
    assert torch.isfinite(decode(res).float()).all()
    over = pa.Stream(st.ctx_len + 1, 1, st.row_offset, st.first_pos + 1,
                     page_table=st.page_table, layout=st.layout)
    assert torch.isnan(decode(res, streams=[over]).float()).any()


def test_hbm_read_probe_reads_every_chunk_once():
    """The read probe folds every 16-byte chunk into its sink exactly once:
    its sink equals the XOR of all 32-bit words of the buffer (a chunk read
    twice would cancel out, a chunk skipped would be missing), for a size
    whose workgroup runs end in part of a step and leave a remainder past the
    last run."""
    g = torch.Generator().manual_seed(77)
    nbytes = 16 * (1024 * 2048 * 3 + 1024 * 700 + 33)
    host = torch.randint(-2**31, 2**31 - 1, (nbytes // 4,), dtype=torch.int32, generator=g)
    buf = host.cuda()
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    pa.hbm_read_probe(buf, sink)
    torch.cuda.synchronize()
    want = np.bitwise_xor.reduce(host.numpy().view(np.uint32))
    assert int(sink.cpu().numpy().view(np.uint32)[0]) == int(want)

