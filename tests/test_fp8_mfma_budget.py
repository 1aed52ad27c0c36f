"""Error budget of fp8 matrix-core products against the float64 oracle, on
fp8-KV workloads shaped like the decode and verify batches.

An fp8 MFMA multiplies E4M3 codes only, so Q (for Q.K^T) and P (for P.V)
must be rounded to E4M3 as well; the stored fp8 K and V are used as they
are.  The oracle reads the stored codes exactly; the emulation here adds
only the extra rounding such a kernel needs:
  * single term: Q per (row, head) scaled by max|q|/448 into E4M3, and P
    (in (0, 1] after the exact max) scaled by 448.  Each alone costs about
    0.023-0.032 of normalised error and both together 0.036-0.037, over the
    3e-2 bound;
  * two terms: x = hi + lo with hi = E4M3(x) and lo = E4M3(x - hi), Q first
    scaled per (row, head) by a power of two that puts max|q| at most 448,
    P (in (0, 1] after the exact max) scaled by 2^4, as the fp8 verify
    kernel scales it (a running max that lags the true one by up to 4 in
    log2 units only raises p, up to 2^8).  Two codes carry 8 significant
    bits, about bf16's precision: the error is 0.7e-3 to 3e-3 (2^6 would
    give 0.6e-3 to 1.1e-3, at the price of a lag of only 2, which moves
    some running max of a 96-column tile in about half of all 64-key
    steps).  Unscaled, the small weights fall into E4M3's subnormal range
    and the error reaches 1e-2 and more.
This file pins these measurements."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import workloads
from tests._util import oracle_logical

FP8_TOL = 3e-2


def _e4m3(x, scale=1.0):
    """Round to E4M3FN codes at `scale` (RNE, saturating) and decode."""
    return oracle.e4m3_to_f64(oracle.e4m3_encode(np.asarray(x, np.float32), scale)) * scale


def _two_term(x, sigma=1.0):
    """hi + lo, each an E4M3 value, of x * sigma (sigma a power of two), / sigma."""
    xs = np.asarray(x, np.float64) * sigma
    hi = _e4m3(xs)
    lo = _e4m3(xs - hi)
    return (hi + lo) / sigma


def _budget(wl, rows):
    from tests._util import bits16
    st = wl.streams[0]
    k8, v8 = oracle_logical(wl, 0)
    K = oracle.e4m3_to_f64(k8) * wl.k_scale
    V = oracle.e4m3_to_f64(v8) * wl.v_scale
    qb = bits16(wl.q[st.row_offset:st.row_offset + st.n_rows])
    Q = oracle.bf16_to_f64(qb)
    G = wl.n_q_heads // wl.n_kv_heads
    ref = oracle.attention(k8, v8, oracle.DTYPE_E4M3, qb, st.first_pos, wl.n_kv_heads,
                           st.ctx_len, rows=np.array(rows, np.int32), sm_scale=wl.sm_scale,
                           k_scale=wl.k_scale, v_scale=wl.v_scale)
    # name -> (how Q is rounded, how P is rounded)
    variants = {"q": ("one", None), "p": (None, "one"), "qp": ("one", "one"),
                "q2": ("two", None), "p2": (None, "two"), "q2p2": ("two", "two"),
                "p2u": (None, "two-unscaled")}
    got = {k: [] for k in variants}
    for r in rows:
        pos = st.first_pos + r
        per = {k: [] for k in variants}
        for h in range(wl.n_q_heads):
            q = Q[r, h]
            Kg, Vg = K[:pos + 1, h // G], V[:pos + 1, h // G]
            qmax = np.abs(q).max()
            sigma = 2.0 ** np.floor(np.log2(448.0 / qmax))
            qr = {None: q, "one": _e4m3(q, qmax / 448), "two": _two_term(q, sigma)}
            for name, (qm, pm) in variants.items():
                z = wl.sm_scale * (Kg @ qr[qm])
                p = np.exp(z - z.max())
                l = p.sum()
                if pm == "one":
                    p = _e4m3(p * 448) / 448
                elif pm == "two":
                    p = _two_term(p, 16.0)
                elif pm == "two-unscaled":
                    p = _two_term(p)
                per[name].append(p @ Vg / l)
        for k in got:
            got[k].append(np.stack(per[k]))
    return {k: oracle.normalised_error(np.stack(v), ref) for k, v in got.items()}


@pytest.mark.parametrize("ctx,n_rows,rows,seed", [(8192, 1, [0], 1003), (20000, 16, [0, 15], 1005)])
def test_fp8_products_one_term_exceed_two_terms_fit(ctx, n_rows, rows, seed):
    wl = workloads.build("budget", n_q_heads=24, n_kv_heads=4, head_dim=256, kv_dtype="fp8",
                         ctx_lens=[ctx], n_rows=[n_rows], seed=seed)
    e = _budget(wl, rows)
    print({k: round(v, 5) for k, v in e.items()})
    # one quantised operand alone already takes at least half of the budget
    # (on the verify rows it can exceed it) ...
    assert e["q"] > FP8_TOL / 2 and e["p"] > FP8_TOL / 2
    # ... and both together are over it
    assert e["qp"] > FP8_TOL
    # two E4M3 terms per operand (P scaled by 2^4) keep the error about an
    # order of magnitude below the tolerance; bf16 Q splits exactly
    assert e["q2"] <= 1e-5
    assert e["p2"] <= 4e-3 and e["q2p2"] <= 4e-3
    # without the scale the weights lose their low bits in the subnormals
    assert e["p2u"] > 5 * e["p2"]


def test_two_term_split_is_exact_for_bf16_inputs_in_range():
    """A bf16 value has 8 significant bits; hi takes the top 4 and lo the
    rest, so hi + lo reproduces every bf16 value whose residual stays in
    E4M3's normal range exactly (checked over every bf16 value in
    [2^-2, 2^8) of both signs)."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    x = oracle.bf16_to_f64(bits)
    sel = np.isfinite(x) & (np.abs(x) >= 0.25) & (np.abs(x) < 256)
    x = x[sel]
    assert np.array_equal(_two_term(x), x)
