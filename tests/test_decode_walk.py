"""CPU model of the register-streaming decode kernel's page walk.

The partial kernel's four waves take the pages of each split round-robin,
read through a rotation by the split index, with one workgroup covering
splits_per_wg consecutive splits.  This file restates that index arithmetic
(sub / phys / advance of the kernel) in Python and checks, for whole and
short last splits and one to three splits per workgroup, that:
  * every (page, chunk) of every split is visited by exactly one wave;
  * the rotation maps each split's pages onto themselves;
  * the page count of the rotation is at least 1 on every call, including
    the look-ahead calls past the last page whose result is discarded.
"""
from __future__ import annotations

import pytest

PAGE = 256
NW = 4


def walk(n_keys, split_keys, spw, split0, chunk_keys):
    """Visits [(wave, physical page, chunk start)] and every np used."""
    n_splits = -(-n_keys // split_keys)
    n_sub = min(spw, n_splits - split0)
    k_lo = split0 * split_keys
    k_hi = min(k_lo + n_sub * split_keys, n_keys)
    p_lo, p_hi = k_lo // PAGE, -(-k_hi // PAGE)
    pps = split_keys // PAGE
    nps = []

    def sub(p):
        return (p - p_lo) // pps

    def phys(p):
        sb = sub(p)
        base = p_lo + sb * pps
        np_ = max(1, min(pps, p_hi - base))
        nps.append(np_)
        v = p - base + (split0 + sb) % np_
        if v >= np_:
            v -= np_
        return base + v

    def advance(p, c0):
        c0 += chunk_keys
        if c0 >= min(PAGE, k_hi - phys(p) * PAGE):
            return p + NW, 0
        return p, c0

    visits = []
    for w in range(NW):
        p, c0 = p_lo + w, 0
        while p < p_hi:
            visits.append((w, phys(p), c0))
            p, c0 = advance(p, c0)
            # the kernel looks two chunks ahead of the one it computes; past
            # the last page these calls' results are discarded
            advance(*advance(p, c0))
    return visits, nps, (p_lo, p_hi, k_hi, n_sub)


@pytest.mark.parametrize("chunk_keys", [32, 64])
@pytest.mark.parametrize("spw", [1, 2, 3])
@pytest.mark.parametrize("n_keys", [4096 * 4, 4096 * 3 + 700, 4096 + 1, 1024 * 5 + 256, 300])
@pytest.mark.parametrize("split_keys", [1024, 4096])
def test_walk_covers_each_split_once(split_keys, n_keys, spw, chunk_keys):
    n_splits = -(-n_keys // split_keys)
    if spw > 1 and split_keys % (NW * PAGE):
        pytest.skip("grouping needs a split's pages to divide over the waves")
    for split0 in range(0, n_splits, spw):
        visits, nps, (p_lo, p_hi, k_hi, n_sub) = walk(n_keys, split_keys, spw, split0,
                                                       chunk_keys)
        assert min(nps) >= 1
        seen = sorted((p, c) for _, p, c in visits)
        want = sorted((p, c) for p in range(p_lo, p_hi)
                      for c in range(0, min(PAGE, k_hi - p * PAGE), chunk_keys))
        assert seen == want
        # with several splits per workgroup, wave w meets the same pages of each
        # split as a workgroup of that split alone would give it
        if n_sub > 1:
            pps = split_keys // PAGE
            for j in range(n_sub):
                alone, _, _ = walk(n_keys, split_keys, 1, split0 + j, chunk_keys)
                lo, hi = p_lo + j * pps, p_lo + (j + 1) * pps
                grouped = sorted(v for v in visits if lo <= v[1] < hi)
                assert grouped == sorted(alone)
