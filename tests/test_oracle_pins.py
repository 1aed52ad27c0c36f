"""Pins for the float64 oracle: each check ties the oracle to something other
than itself -- a library routine (torch's float8/bf16 casts, torch's
scaled_dot_product_attention in float64), a closed form, an invariant, or a
fixture worked by hand from the pages' address formula.  CPU only."""
from __future__ import annotations

import json
import math
import random
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import workloads
from tests._util import bits16

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
PAGE = 256


# ----------------------------------------------------------------------------- codecs

def test_e4m3_decode_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.e4m3_to_f64(codes)
    ref = torch.from_numpy(codes.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])
    # E4M3FN facts: largest finite 448, smallest subnormal 2^-9, NaN only at S.1111.111
    assert ours[0x7E] == 448.0 and ours[0x01] == 2.0 ** -9 and ours[0x08] == 2.0 ** -6
    assert np.isnan(ours[0x7F]) and np.isnan(ours[0xFF]) and np.isnan(ours).sum() == 2


def test_bf16_decode_all_patterns_match_torch():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = oracle.bf16_to_f64(bits)
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64)
    ref = ref.numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])


def _torch_quant(x32: np.ndarray, scale: float) -> np.ndarray:
    t = torch.from_numpy(x32) / torch.tensor(scale, dtype=torch.float32)
    t = torch.clamp(t, -448.0, 448.0)
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


@pytest.mark.parametrize("scale", [1.0, 0.0107421875, 3.7, 1.0 / 448.0 * 4.75])
def test_e4m3_encode_every_bf16_value_matches_torch(scale):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    x = oracle.bf16_to_f64(bits).astype(np.float32)
    x = x[np.isfinite(x)]
    ours = oracle.e4m3_encode(x, scale)
    ref = _torch_quant(x, np.float32(scale))
    assert np.array_equal(ours, ref)


def test_e4m3_encode_ties_round_to_even():
    vals = oracle.e4m3_to_f64(np.arange(0, 0x7F, dtype=np.uint8))  # 0 .. 448, ascending
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)
    assert np.array_equal(mids.astype(np.float64), (vals[:-1] + vals[1:]) / 2)  # exact ties
    got = oracle.e4m3_encode(mids, 1.0)
    lo = np.arange(0, 0x7E, dtype=np.uint8)
    want = np.where(lo % 2 == 0, lo, lo + 1).astype(np.uint8)  # even mantissa wins
    assert np.array_equal(got, want)
    assert np.array_equal(oracle.e4m3_encode(-mids, 1.0), want | 0x80)
    assert np.array_equal(got, _torch_quant(mids, 1.0))
    # saturation instead of NaN above the largest finite value
    big = np.array([448.0, 463.9, 464.0, 480.0, 1e6, -1e6], np.float32)
    assert list(oracle.e4m3_encode(big, 1.0)) == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE]


# ----------------------------------------------------------------------------- addressing

def test_store_matches_hand_worked_page_addresses():
    g = json.load(open(os.path.join(GOLDEN, "page_addresses.json")))
    D, H, PS = g["head_dim"], g["n_kv_heads"], g["page_stride"]
    pt = np.array(g["page_table"], np.int32)
    n_pos = PAGE * len(pt)
    pool_k = np.zeros(8 * PS, np.uint16)
    pool_v = np.zeros(8 * PS, np.uint16)
    # row r, head h, dim d carries the tag (r * H + h) * D + d + 1 (all distinct, < 2^16)
    tags = (np.arange(n_pos * H * D, dtype=np.uint32) + 1).astype(np.uint16)
    rows = tags.reshape(n_pos, H, D)
    oracle.store(pool_k, pool_v, oracle.DTYPE_BF16, rows, rows, 0, page_table=pt, page_stride=PS)
    for c in g["cases"]:
        want = rows[c["pos"], c["kv_head"]]
        assert np.array_equal(pool_k[c["offset"]:c["offset"] + D], want), c
        assert np.array_equal(pool_v[c["offset"]:c["offset"] + D], want), c


# ----------------------------------------------------------------------------- attention

def _rand_case(rng, hq, hkv, d, ctx, n_rows, fp8=False):
    q = torch.from_numpy(rng.standard_normal((n_rows, hq, d)).astype(np.float32)).bfloat16()
    k = torch.from_numpy(rng.standard_normal((ctx, hkv, d)).astype(np.float32)).bfloat16()
    v = torch.from_numpy(rng.standard_normal((ctx, hkv, d)).astype(np.float32)).bfloat16()
    return q, k, v


def _sdpa(q64, k64, v64, positions, scale):
    """torch.nn.functional.scaled_dot_product_attention in float64 with an
    explicit boolean mask (key t visible to a row at position p iff t <= p)
    and torch's own grouped-query head mapping."""
    t = k64.shape[0]
    mask = torch.arange(t)[None, :] <= torch.as_tensor(positions)[:, None]
    out = F.scaled_dot_product_attention(q64.transpose(0, 1), k64.transpose(0, 1),
                                         v64.transpose(0, 1), attn_mask=mask, scale=scale,
                                         enable_gqa=True)
    return out.transpose(0, 1).numpy()


CASES = [  # (Hq, Hkv, D, ctx, n_rows)
    (4, 2, 16, 1, 1), (4, 2, 16, 255, 3), (4, 2, 32, 256, 1), (6, 1, 16, 257, 5),
    (6, 1, 32, 600, 17), (4, 2, 32, 513, 40),
]


@pytest.mark.parametrize("hq,hkv,d,ctx,n_rows", CASES)
@pytest.mark.parametrize("paged", [False, True])
def test_attention_matches_torch_sdpa_bf16(hq, hkv, d, ctx, n_rows, paged):
    rng = np.random.default_rng(hash((hq, hkv, d, ctx, n_rows)) % 2 ** 32)
    q, k, v = _rand_case(rng, hq, hkv, d, ctx, n_rows)
    first = ctx - n_rows
    if paged:
        n_pages = math.ceil(ctx / PAGE) + 2
        pt = rng.permutation(n_pages).astype(np.int32)[:math.ceil(ctx / PAGE)]
        ps = hkv * PAGE * d
        kp = np.zeros(n_pages * ps, np.uint16)
        vp = np.zeros(n_pages * ps, np.uint16)
        oracle.store(kp, vp, oracle.DTYPE_BF16, bits16(k), bits16(v), 0, page_table=pt,
                     page_stride=ps)
        got = oracle.attention(kp, vp, oracle.DTYPE_BF16, bits16(q), first, hkv, ctx,
                               page_table=pt, page_stride=ps)
    else:
        got = oracle.attention(bits16(k), bits16(v), oracle.DTYPE_BF16, bits16(q), first, hkv, ctx)
    ref = _sdpa(q.double(), k.double(), v.double(), np.arange(first, ctx), 1.0 / math.sqrt(d))
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("hq,hkv,d,ctx,n_rows", CASES[1::2])
def test_attention_matches_torch_sdpa_fp8(hq, hkv, d, ctx, n_rows):
    rng = np.random.default_rng(7 + ctx)
    q, k, v = _rand_case(rng, hq, hkv, d, ctx, n_rows)
    ks = float(k.float().abs().max()) / 448
    vs = float(v.float().abs().max()) / 448
    kc = np.zeros((ctx, hkv, d), np.uint8)
    vc = np.zeros_like(kc)
    oracle.store(kc, vc, oracle.DTYPE_E4M3, bits16(k), bits16(v), 0, k_scale=ks, v_scale=vs)
    got = oracle.attention(kc, vc, oracle.DTYPE_E4M3, bits16(q), ctx - n_rows, hkv, ctx,
                           k_scale=ks, v_scale=vs)
    # library path: torch's own e4m3fn decode of the stored codes, times the scale
    k64 = torch.from_numpy(kc).view(torch.float8_e4m3fn).double() * ks
    v64 = torch.from_numpy(vc).view(torch.float8_e4m3fn).double() * vs
    ref = _sdpa(q.double(), k64, v64, np.arange(ctx - n_rows, ctx), 1.0 / math.sqrt(d))
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def test_zero_query_gives_running_mean_of_values():
    # Q = 0: every visible key has the same logit, so row p returns mean(V[0..p]);
    # pins the causal boundary (inclusive of the row's own position).
    rng = np.random.default_rng(3)
    hq, hkv, d, ctx, n = 4, 2, 16, 300, 30
    _, k, v = _rand_case(rng, hq, hkv, d, ctx, n)
    q = torch.zeros((n, hq, d), dtype=torch.bfloat16)
    got = oracle.attention(bits16(k), bits16(v), oracle.DTYPE_BF16, bits16(q), ctx - n, hkv, ctx)
    vd = v.double().numpy()
    for i in range(n):
        p = ctx - n + i
        mean = vd[:p + 1].mean(axis=0)  # [Hkv][D]
        for h in range(hq):
            np.testing.assert_allclose(got[i, h], mean[h // (hq // hkv)], rtol=0, atol=1e-13)


def test_constant_value_per_kv_head_pins_group_map():
    # V[t, g, :] = g  =>  out[h] = the kv head h reads = floor(h / G)
    rng = np.random.default_rng(4)
    hq, hkv, d, ctx = 12, 4, 16, 520
    q, k, _ = _rand_case(rng, hq, hkv, d, ctx, 3)
    v = torch.arange(hkv, dtype=torch.float32)[None, :, None].expand(ctx, hkv, d).bfloat16()
    got = oracle.attention(bits16(k), bits16(v), oracle.DTYPE_BF16, bits16(q), ctx - 3, hkv, ctx)
    for h in range(hq):
        np.testing.assert_allclose(got[:, h], h // 3, rtol=0, atol=1e-13)


def test_single_key_returns_its_value():
    rng = np.random.default_rng(5)
    q, k, v = _rand_case(rng, 4, 2, 32, 1, 1)
    got = oracle.attention(bits16(k), bits16(v), oracle.DTYPE_BF16, bits16(q), 0, 2, 1)
    for h in range(4):
        np.testing.assert_array_equal(got[0, h], v[0, h // 2].double().numpy())


def test_equal_keys_give_uniform_mean():
    rng = np.random.default_rng(6)
    hq, hkv, d, ctx = 4, 2, 16, 77
    q, _, v = _rand_case(rng, hq, hkv, d, ctx, 1)
    k = torch.from_numpy(rng.standard_normal((1, hkv, d)).astype(np.float32)).bfloat16()
    k = k.expand(ctx, hkv, d).contiguous()
    got = oracle.attention(bits16(k), bits16(v), oracle.DTYPE_BF16, bits16(q), ctx - 1, hkv, ctx)
    mean = v.double().numpy().mean(axis=0)
    for h in range(hq):
        np.testing.assert_allclose(got[0, h], mean[h // 2], rtol=0, atol=1e-13)


def test_dominant_aligned_key_returns_its_value():
    # one key parallel to q with a huge logit: softmax collapses onto it
    hq, hkv, d, ctx = 2, 1, 16, 40
    rng = np.random.default_rng(8)
    _, k, v = _rand_case(rng, hq, hkv, d, ctx, 1)
    k = k * 0.01
    q = torch.zeros((1, hq, d), dtype=torch.bfloat16)
    q[0, :, 0] = 64.0
    k[17, 0, :] = 0
    k[17, 0, 0] = 64.0   # logit 64*64/4 = 1024 vs ~0 for the others
    got = oracle.attention(bits16(k), bits16(v), oracle.DTYPE_BF16, bits16(q), ctx - 1, hkv, ctx)
    for h in range(hq):
        np.testing.assert_allclose(got[0, h], v[17, 0].double().numpy(), rtol=0, atol=1e-12)


# ----------------------------------------------------------------------------- invariants

def test_permuted_pool_equals_unpaged_bitwise_and_swap_differs():
    rng = np.random.default_rng(9)
    hq, hkv, d, ctx, n = 6, 2, 32, 1100, 4
    q, k, v = _rand_case(rng, hq, hkv, d, ctx, n)
    n_used = math.ceil(ctx / PAGE)
    n_pages = n_used + 3
    pt = rng.permutation(n_pages).astype(np.int32)[:n_used]
    ps = hkv * PAGE * d
    kp = np.zeros(n_pages * ps, np.uint16)
    vp = np.zeros_like(kp)
    oracle.store(kp, vp, oracle.DTYPE_BF16, bits16(k), bits16(v), 0, page_table=pt, page_stride=ps)
    unused = sorted(set(range(n_pages)) - set(pt.tolist()))
    filler = rng.standard_normal((PAGE, hkv, d)).astype(np.float32)
    oracle.store(kp, vp, oracle.DTYPE_BF16, bits16(torch.from_numpy(filler).bfloat16()),
                 bits16(torch.from_numpy(filler).bfloat16()), 0,
                 page_table=np.array(unused[:1], np.int32), page_stride=ps)
    paged = oracle.attention(kp, vp, oracle.DTYPE_BF16, bits16(q), ctx - n, hkv, ctx,
                             page_table=pt, page_stride=ps)
    flat = oracle.attention(bits16(k), bits16(v), oracle.DTYPE_BF16, bits16(q), ctx - n, hkv, ctx)
    assert np.array_equal(paged, flat)  # same values in the same order: bitwise equal
    bad = pt.copy()
    bad[1] = unused[0]  # a page of another stream in place of the stream's own
    swapped = oracle.attention(kp, vp, oracle.DTYPE_BF16, bits16(q), ctx - n, hkv, ctx,
                               page_table=bad, page_stride=ps)
    assert oracle.normalised_error(swapped, flat) > 0.05


@pytest.mark.parametrize("split", [64, 256, 4096])
def test_split_then_merge_equals_direct(split):
    rng = np.random.default_rng(10 + split)
    hq, hkv, d, ctx, n = 6, 2, 32, 700, 70
    q, k, v = _rand_case(rng, hq, hkv, d, ctx, n)
    first = ctx - n
    n_split = math.ceil(ctx / split)
    m, l, o = oracle.attention_split(bits16(k), bits16(v), oracle.DTYPE_BF16, bits16(q), first,
                                     hkv, ctx, split, n_split)
    if split == 64:  # rows before the last split's start see a wholly masked last split
        assert np.isneginf(m[0, :, -1]).all() and (l[0, :, -1] == 0).all()
    merged = oracle.merge(m, l, o)
    direct = oracle.attention(bits16(k), bits16(v), oracle.DTYPE_BF16, bits16(q), first, hkv, ctx)
    np.testing.assert_allclose(merged, direct, rtol=1e-13, atol=1e-14)


def test_sampled_rows_equal_full_rows():
    rng = np.random.default_rng(11)
    q, k, v = _rand_case(rng, 4, 2, 16, 400, 50)
    full = oracle.attention(bits16(k), bits16(v), oracle.DTYPE_BF16, bits16(q), 350, 2, 400)
    sel = np.array([0, 7, 49, 13], np.int32)
    part = oracle.attention(bits16(k), bits16(v), oracle.DTYPE_BF16, bits16(q), 350, 2, 400,
                            rows=sel, n_threads=3)
    assert np.array_equal(part, full[sel])


def test_row_past_stored_keys_is_refused():
    rng = np.random.default_rng(12)
    q, k, v = _rand_case(rng, 4, 2, 16, 10, 2)
    with pytest.raises(ValueError):
        oracle.attention(bits16(k), bits16(v), oracle.DTYPE_BF16, bits16(q), 9, 2, 10)


# ----------------------------------------------------------------------------- draft-tree rows

def _tree_mask(parents, first, ctx):
    """Visibility from the parent list itself (walking up to the prefix):
    row i sees every key before `first` and the keys of itself and its
    ancestors -- an independent statement of the ancestor-table rule."""
    n = len(parents)
    mask = np.zeros((n, ctx), bool)
    mask[:, :first] = True
    for i in range(n):
        j = i
        while j >= 0:
            mask[i, first + j] = True
            j = parents[j]
    return torch.from_numpy(mask)


def _sdpa_mask(q64, k64, v64, mask, scale):
    out = F.scaled_dot_product_attention(q64.transpose(0, 1), k64.transpose(0, 1),
                                         v64.transpose(0, 1), attn_mask=mask, scale=scale,
                                         enable_gqa=True)
    return out.transpose(0, 1).numpy()


@pytest.mark.parametrize("seed,n_rows,ctx", [(1, 1, 40), (2, 5, 300), (3, 16, 700), (4, 32, 1000)])
@pytest.mark.parametrize("paged", [False, True])
def test_tree_rows_match_sdpa_with_ancestor_mask(seed, n_rows, ctx, paged):
    rng = np.random.default_rng(100 + seed)
    hq, hkv, d = 6, 2, 32
    q, k, v = _rand_case(rng, hq, hkv, d, ctx, n_rows)
    first = ctx - n_rows
    parents = workloads.random_parents(n_rows, random.Random(seed))
    words = workloads.tree_words(parents)
    if paged:
        n_pages = math.ceil(ctx / PAGE) + 1
        pt = rng.permutation(n_pages).astype(np.int32)[:math.ceil(ctx / PAGE)]
        ps = hkv * PAGE * d
        kp = np.zeros(n_pages * ps, np.uint16)
        vp = np.zeros(n_pages * ps, np.uint16)
        oracle.store(kp, vp, oracle.DTYPE_BF16, bits16(k), bits16(v), 0, page_table=pt,
                     page_stride=ps)
        got = oracle.attention(kp, vp, oracle.DTYPE_BF16, bits16(q), first, hkv, ctx,
                               page_table=pt, page_stride=ps, tree=words)
    else:
        got = oracle.attention(bits16(k), bits16(v), oracle.DTYPE_BF16, bits16(q), first, hkv,
                               ctx, tree=words)
    ref = _sdpa_mask(q.double(), k.double(), v.double(), _tree_mask(parents, first, ctx),
                     1.0 / math.sqrt(d))
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def test_tree_fp8_rows_match_sdpa_with_ancestor_mask():
    rng = np.random.default_rng(120)
    hq, hkv, d, ctx, n = 4, 1, 32, 500, 9
    q, k, v = _rand_case(rng, hq, hkv, d, ctx, n)
    ks = float(k.float().abs().max()) / 448
    vs = float(v.float().abs().max()) / 448
    kc = np.zeros((ctx, hkv, d), np.uint8)
    vc = np.zeros_like(kc)
    oracle.store(kc, vc, oracle.DTYPE_E4M3, bits16(k), bits16(v), 0, k_scale=ks, v_scale=vs)
    parents = [-1, 0, 0, 1, 1, 2, -1, 6, 3]  # two roots on the prefix
    got = oracle.attention(kc, vc, oracle.DTYPE_E4M3, bits16(q), ctx - n, hkv, ctx, k_scale=ks,
                           v_scale=vs, tree=workloads.tree_words(parents))
    k64 = torch.from_numpy(kc).view(torch.float8_e4m3fn).double() * ks
    v64 = torch.from_numpy(vc).view(torch.float8_e4m3fn).double() * vs
    ref = _sdpa_mask(q.double(), k64, v64, _tree_mask(parents, ctx - n, ctx), 1.0 / math.sqrt(d))
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def test_chain_tree_is_exactly_the_causal_rows_and_high_bits_are_ignored():
    rng = np.random.default_rng(121)
    q, k, v = _rand_case(rng, 6, 2, 32, 600, 16)
    causal = oracle.attention(bits16(k), bits16(v), oracle.DTYPE_BF16, bits16(q), 584, 2, 600)
    chain = workloads.tree_words(list(range(-1, 15)))
    assert np.array_equal(chain, (1 << np.arange(1, 17, dtype=np.uint64)) - 1)
    got = oracle.attention(bits16(k), bits16(v), oracle.DTYPE_BF16, bits16(q), 584, 2, 600,
                           tree=chain)
    assert np.array_equal(got, causal)
    # bits above a row's own index name later rows: they are ignored
    noisy = chain | np.uint32(0xFFFF0000)
    got2 = oracle.attention(bits16(k), bits16(v), oracle.DTYPE_BF16, bits16(q), 584, 2, 600,
                            tree=noisy)
    assert np.array_equal(got2, causal)


def test_tree_split_then_merge_equals_direct_and_rows_over_32_are_refused():
    rng = np.random.default_rng(122)
    hq, hkv, d, ctx, n = 6, 2, 32, 4100, 16
    q, k, v = _rand_case(rng, hq, hkv, d, ctx, n)
    words = workloads.tree_words(workloads.random_parents(n, random.Random(5)))
    m, l, o = oracle.attention_split(bits16(k), bits16(v), oracle.DTYPE_BF16, bits16(q), ctx - n,
                                     hkv, ctx, 1024, 5, tree=words)
    direct = oracle.attention(bits16(k), bits16(v), oracle.DTYPE_BF16, bits16(q), ctx - n, hkv,
                              ctx, tree=words)
    np.testing.assert_allclose(oracle.merge(m, l, o), direct, rtol=1e-13, atol=1e-14)
    q33, k33, v33 = _rand_case(rng, 2, 1, 16, 100, 33)
    with pytest.raises(ValueError):
        oracle.attention(bits16(k33), bits16(v33), oracle.DTYPE_BF16, bits16(q33), 67, 1, 100,
                         tree=np.ones(33, np.uint32))
