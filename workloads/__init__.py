"""Seeded synthetic workloads for paged grouped-query attention.

This module only draws inputs: random numbers, page permutations, context
lengths and per-tensor fp8 scales.  It holds none of the attention
arithmetic, and both the HIP path's tests and the oracle read the same
arrays from it.

Recipe (every config):
  * ``g = torch.Generator('cpu').manual_seed(seed)`` with seed = 1000 + the
    config number;
  * draw order: the page permutation, then Q ``[rows][Hq][D]``, then for
    each stream in order K ``[ctx][Hkv][D]`` and V ``[ctx][Hkv][D]``, then the
    filler rows of unused pool pages; all N(0, 1) in float32, rounded to
    bf16 by torch (round to nearest even);
  * context lengths (mixed batch) come from ``random.Random(seed)``;
  * fp8 caches use per-tensor scales ``max|K| / 448`` and ``max|V| / 448``
    over every stream's unquantised bf16 rows, computed once, so that alone
    and batched runs see the same codes.
"""
from __future__ import annotations

import math
import random
from dataclasses import dataclass, field

import numpy as np
import torch

PAGE = 256
E4M3_MAX = 448.0


@dataclass
class StreamSpec:
    layout: str            # "paged" or "slab"
    ctx_len: int           # positions stored for the stream
    n_rows: int            # query rows in the launch
    first_pos: int         # absolute position of the first query row
    row_offset: int        # index of the stream's first row in Q / out
    pages: np.ndarray | None = None   # int32 page ids, ceil(ctx_len / 256) of them
    slab_cap: int = 0      # slab capacity in positions (slab layout)
    tree: np.ndarray | None = None    # uint32 ancestor word per row, or None (causal)


@dataclass
class Workload:
    name: str
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    kv_dtype: str          # "bf16" or "fp8"
    n_pages: int
    streams: list
    q: torch.Tensor        # bf16 [total_rows][Hq][D]
    k_rows: list           # per stream bf16 [ctx][Hkv][D]
    v_rows: list
    filler_pages: np.ndarray        # int32 ids of pool pages no stream uses
    filler_k: torch.Tensor | None   # bf16 [len(filler_pages)*256][Hkv][D]
    filler_v: torch.Tensor | None
    sm_scale: float
    split_keys: int = 4096
    k_scale: float = 1.0
    v_scale: float = 1.0
    seed: int = 0
    meta: dict = field(default_factory=dict)

    @property
    def total_rows(self) -> int:
        return int(self.q.shape[0])


def _bf16(shape, g):
    return torch.randn(shape, generator=g, dtype=torch.float32).to(torch.bfloat16)


def _scales(ws: list, kind: str) -> float:
    m = 0.0
    for t in ws:
        if t is not None and t.numel():
            m = max(m, float(t.float().abs().max()))
    return m / E4M3_MAX if m > 0 else 1.0


def tree_words(parents) -> np.ndarray:
    """Ancestor words of a draft tree given in topological order: parents[i]
    is the row of node i's parent (< i), or -1 for a node whose parent is the
    committed prefix.  Bit j of word i is set when row j is node i or one of
    its ancestors."""
    words = []
    for i, p in enumerate(parents):
        if not (-1 <= p < i):
            raise ValueError("parents must precede their children")
        words.append((words[p] if p >= 0 else 0) | (1 << i))
    return np.asarray(words, dtype=np.uint32)


def random_parents(n: int, rng: random.Random) -> list:
    """A random draft tree over n rows: node 0 hangs off the prefix, every
    later node off a uniformly drawn earlier node."""
    return [-1] + [rng.randrange(i) for i in range(1, n)]


def build(name: str, *, n_q_heads: int, n_kv_heads: int, head_dim: int, kv_dtype: str,
          ctx_lens: list, n_rows: list, layouts: list | None = None, n_pages: int | None = None,
          seed: int = 0, split_keys: int = 4096, fill_unused: bool = True,
          sm_scale: float | None = None, slab_cap: int | None = None,
          trees: list | None = None) -> Workload:
    """Generic generator: one stream per entry of ``ctx_lens``; stream s has
    ``n_rows[s]`` query rows at its last positions ``ctx-n..ctx-1``.
    ``trees[s]`` (optional): None (causal rows), "chain" (the causal chain as
    an explicit ancestor table), "random" (a random draft tree drawn from
    ``random.Random(seed + 7)``, after every torch draw) or a parents list."""
    n_streams = len(ctx_lens)
    layouts = layouts or ["paged"] * n_streams
    g = torch.Generator("cpu").manual_seed(seed)
    need = [math.ceil(c / PAGE) for c in ctx_lens]
    paged_need = sum(n for n, lay in zip(need, layouts) if lay == "paged")
    if n_pages is None:
        n_pages = max(paged_need, 1)
    if paged_need > n_pages:
        raise ValueError("pool too small for the paged streams")
    perm = torch.randperm(n_pages, generator=g).numpy().astype(np.int32)
    streams, at, row_off = [], 0, 0
    for s in range(n_streams):
        ctx, r = int(ctx_lens[s]), int(n_rows[s])
        pages = None
        if layouts[s] == "paged":
            pages = perm[at:at + need[s]].copy()
            at += need[s]
        cap = 0
        if layouts[s] == "slab":
            cap = int(slab_cap) if slab_cap else need[s] * PAGE
        streams.append(StreamSpec(layouts[s], ctx, r, ctx - r, row_off, pages, cap))
        row_off += r
    q = _bf16((row_off, n_q_heads, head_dim), g)
    k_rows, v_rows = [], []
    for s in range(n_streams):
        k_rows.append(_bf16((ctx_lens[s], n_kv_heads, head_dim), g))
        v_rows.append(_bf16((ctx_lens[s], n_kv_heads, head_dim), g))
    unused = perm[at:].copy()
    fk = fv = None
    if fill_unused and len(unused):
        fk = _bf16((len(unused) * PAGE, n_kv_heads, head_dim), g)
        fv = _bf16((len(unused) * PAGE, n_kv_heads, head_dim), g)
    if trees is not None:
        trng = random.Random(seed + 7)
        for st, t in zip(streams, trees):
            if t is None:
                continue
            if isinstance(t, str):
                parents = (list(range(-1, st.n_rows - 1)) if t == "chain"
                           else random_parents(st.n_rows, trng))
            else:
                parents = list(t)
            st.tree = tree_words(parents)
    ks = vs = 1.0
    if kv_dtype == "fp8":
        ks = _scales(k_rows, "k")
        vs = _scales(v_rows, "v")
    return Workload(name=name, n_q_heads=n_q_heads, n_kv_heads=n_kv_heads, head_dim=head_dim,
                    kv_dtype=kv_dtype, n_pages=n_pages, streams=streams, q=q, k_rows=k_rows,
                    v_rows=v_rows, filler_pages=unused, filler_k=fk, filler_v=fv,
                    sm_scale=(1.0 / math.sqrt(head_dim)) if sm_scale is None else sm_scale,
                    split_keys=split_keys, k_scale=ks, v_scale=vs, seed=seed)


# ----------------------------------------------------------------------------- the five workloads

def config1() -> Workload:
    """Decode, 1 stream, 1 row: 8 q / 2 kv heads, D 128, context 1,024 in 4
    pages at a seeded permutation of an 8-page pool, bf16."""
    return build("decode-1x1024-h8kv2-d128-bf16", n_q_heads=8, n_kv_heads=2, head_dim=128,
                 kv_dtype="bf16", ctx_lens=[1024], n_rows=[1], n_pages=8, seed=1001)


def config2(ctx: int = 65536, n_streams: int = 8) -> Workload:
    """Decode batch: 8 streams x 1 row at context 65,536, 24 q / 4 kv heads,
    D 256, bf16, pages shuffled in one shared pool, 4,096-key splits."""
    return build(f"decode-{n_streams}x{ctx}-h24kv4-d256-bf16", n_q_heads=24, n_kv_heads=4,
                 head_dim=256, kv_dtype="bf16", ctx_lens=[ctx] * n_streams,
                 n_rows=[1] * n_streams, seed=1002)


def config3(ctx: int = 65536, n_streams: int = 8) -> Workload:
    """As config 2 with fp8-e4m3 KV and per-tensor scales; streams 0-3 paged
    (in a shuffled pool), 4-7 contiguous slabs, in the same launch."""
    half = n_streams // 2
    return build(f"decode-{n_streams}x{ctx}-h24kv4-d256-fp8-mixed", n_q_heads=24, n_kv_heads=4,
                 head_dim=256, kv_dtype="fp8", ctx_lens=[ctx] * n_streams,
                 n_rows=[1] * n_streams, layouts=["paged"] * half + ["slab"] * (n_streams - half),
                 seed=1003)


def config4(prefix: int = 28672, rows: int = 4096) -> Workload:
    """Prefill chunk: 1 stream, 4,096 causal rows after a 28,672-position
    paged prefix, 24 q / 4 kv heads, D 256, bf16."""
    return build(f"prefill-{rows}after{prefix}-h24kv4-d256-bf16", n_q_heads=24, n_kv_heads=4,
                 head_dim=256, kv_dtype="bf16", ctx_lens=[prefix + rows], n_rows=[rows],
                 seed=1004)


def config5_lengths(seed: int = 1005, n_streams: int = 16, lo: int = 4096, hi: int = 110000,
                    pool_pages: int = 5080):
    """Context lengths uniform on [lo, hi] (inclusive), redrawn with seed+1
    if the pages they need exceed the pool."""
    while True:
        rnd = random.Random(seed)
        lens = [rnd.randint(lo, hi) for _ in range(n_streams)]
        if sum(math.ceil(L / PAGE) for L in lens) <= pool_pages:
            return lens, seed
        seed += 1


def config5(n_streams: int = 16, rows: int = 16, lo: int = 4096, hi: int = 110000,
            pool_pages: int = 5080) -> Workload:
    """Mixed verify batch: 16 streams, contexts U[4k, 110k], 16 causal verify
    rows each, 256-position pages in a 1.3M-row pool (5,080 pages, some
    unused), 24 q / 4 kv heads, D 256, fp8-e4m3 with per-tensor scales."""
    lens, seed = config5_lengths(1005, n_streams, lo, hi, pool_pages)
    return build(f"verify-{n_streams}x{rows}-h24kv4-d256-fp8", n_q_heads=24, n_kv_heads=4,
                 head_dim=256, kv_dtype="fp8", ctx_lens=lens, n_rows=[rows] * n_streams,
                 n_pages=pool_pages, seed=seed, fill_unused=False)


CONFIGS = {1: config1, 2: config2, 3: config3, 4: config4, 5: config5}
