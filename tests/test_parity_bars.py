"""CPU checks that the full-size parity bars (``bars.py``) can see a kernel
mistake at tile granularity, and that they leave room for a correct one.

For sampled rows of the full-size workloads:
  * the oracle run with one 32-key tile removed from the keys (what a
    kernel that skipped a K/V tile would return) must fail the bars;
  * an emulation of a correct kernel's rounding (probabilities rounded to
    bf16 before P V, the row sum over the unrounded ones, O rounded to bf16)
    must pass them with a margin.
"""
import numpy as np
import pytest
import torch

import oracle
from bars import SIGMAS, TOL_O, U_BF16, bar_violations, round_bf16, scales_head
from exact_io_aware_attn_amd.inputs import WORKLOADS, make_inputs

pytestmark = pytest.mark.slow


def _rows(w, heads, n_rows=24, seed=0):
    rng = np.random.default_rng(seed)
    rows = np.unique(np.concatenate([[w.Nq - 1], rng.integers(0, w.Nq, n_rows)]))
    return [(b, hq, rows) for b, hq in heads]


def _emulated_kernel(q, k, v, scale, causal, rows):
    """Exact scores; P = exp(s - m) rounded to bf16 for P V; l over the
    unrounded P; O rounded to bf16.  LSE from the same m and l."""
    Nq, Nkv = q.shape[0], k.shape[0]
    S = (q[rows] @ k.T) * scale
    vis = oracle.visible_mask(Nq, Nkv, causal, rows)
    S = np.where(vis, S, -np.inf)
    m = S.max(axis=1)
    P = np.where(vis, np.exp(S - m[:, None]), 0.0)
    l = P.sum(axis=1)
    O = round_bf16((round_bf16(P) @ v) / l[:, None])
    return O, m + np.log(l)


CASES = [
    # (workload, dropped key tile start, heads)
    ("splitd_bf16_d512", 2048, [(0, 0), (0, 5)]),
    ("splitd_bf16_d1024", 1024, [(0, 3)]),
    ("gqa_cross_bf16", 4096, [(0, 0), (1, 31)]),
    ("gqa_causal_bf16", 4096, [(1, 7)]),
]


@pytest.mark.parametrize("name,tile0,heads", CASES, ids=[c[0] for c in CASES])
def test_bars_catch_a_dropped_key_tile(name, tile0, heads):
    w = WORKLOADS[name]
    q, k, v = (t.to(torch.float64).numpy() for t in make_inputs(w))
    G = w.Hq // w.Hkv
    keep = np.ones(w.Nkv, dtype=bool)
    keep[tile0:tile0 + 32] = False
    for b, hq, rows in _rows(w, heads):
        qh, kh, vh = q[b, hq], k[b, hq // G], v[b, hq // G]
        Oref, Lref = oracle.attention_head(qh, kh, vh, w.scale, w.causal, rows=rows)
        sc = scales_head(qh, kh, vh, w.scale, w.causal, rows, Oref, Lref)
        sig = sc["sigma"]
        # a correct kernel's rounding passes, with at least 2x margin on the
        # scale-aware output bar
        Oe, Le = _emulated_kernel(qh, kh, vh, w.scale, w.causal, rows)
        assert bar_violations(Oe, Le, Oref, Lref, "bf16", sc=sc) == []
        assert (np.abs(Oe - Oref) <= 0.5 * (U_BF16 * np.abs(Oref) + SIGMAS * sig)).all()
        # the same rows without one key tile fail; under the causal mask
        # only rows that see the tile are affected, and the sampled set has
        # such rows (the last row sees every key)
        Od, Ld = oracle.attention_head(qh, kh[keep], vh[keep], w.scale, False, rows=rows) if not w.causal \
            else _drop_causal(qh, kh, vh, w.scale, rows, keep)
        bad = bar_violations(Od, Ld, Oref, Lref, "bf16", sc=sc)
        assert any("|dLSE|" in m for m in bad), bad
        if not w.causal:
            # every sampled row sees the tile: the output bar sees it too
            assert any("elements with |dO|" in m for m in bad), bad
        # the stated absolute output bar alone would not have seen it
        assert np.abs(Od - Oref).max() <= TOL_O["bf16"]


def _drop_causal(q, k, v, scale, rows, keep):
    """Causal attention (Nq == Nkv, bottom-right = top-left) with the keys
    outside ``keep`` removed, rows at their absolute positions."""
    Nq, Nkv = q.shape[0], k.shape[0]
    S = (q[rows] @ k.T) * scale
    vis = oracle.visible_mask(Nq, Nkv, True, rows) & keep[None, :]
    from oracle.exact import masked_softmax_pv
    return masked_softmax_pv(S, vis, v)


def _fp8_scores_truncated(qc, kc):
    """Dot products of e4m3 code values as the fp8 matrix instruction forms
    them (measured on gfx950): groups of 8 consecutive indices, each product
    of a group truncated toward zero to a multiple of 2^(e - 13), e the
    exponent of the group's largest product, which itself stays exact."""
    R, K = qc.shape
    out = np.empty((R, kc.shape[0]))
    kg = kc.reshape(kc.shape[0], K // 8, 8)
    for i in range(R):
        prod = qc[i].reshape(1, K // 8, 8) * kg
        mx = np.abs(prod).max(axis=2, keepdims=True)
        e = np.floor(np.log2(np.where(mx > 0, mx, 1.0)))
        quantum = np.exp2(e - 13)
        t = np.trunc(prod / quantum) * quantum
        t = np.where(np.abs(prod) == mx, prod, t)
        out[i] = t.sum(axis=(1, 2))
    return out


def test_bar_holds_emulated_rounding_on_outlier_inputs():
    """e4m3 inputs with 1% outlier channels (the shape whose rows include
    near-cancelling outputs): an emulated correct kernel passes the bars
    with a 2x margin on the output bar, and one whose scores carry the fp8
    matrix instruction's grouped truncation passes the bars that account
    for it."""
    from exact_io_aware_attn_amd.inputs import Workload
    w = Workload("fp8small", 1, 4, 1, 700, 1000, 128, False, "fp8", seed=7, outlier_frac=0.01)
    q8, k8, v8, desc = make_inputs(w)
    q, k, v = (oracle.e4m3fn_decode(t.view(torch.uint8).numpy()) * np.float64(d) for t, d in zip((q8, k8, v8), desc))
    rows = np.arange(w.Nq)
    for hq in range(w.Hq):
        Oref, Lref = oracle.attention_head(q[0, hq], k[0, 0], v[0, 0], w.scale, False)
        sc = scales_head(q[0, hq], k[0, 0], v[0, 0], w.scale, False, rows, Oref, Lref)
        sig = sc["sigma"]
        Oe, Le = _emulated_kernel(q[0, hq], k[0, 0], v[0, 0], w.scale, False, rows)
        assert bar_violations(Oe, Le, Oref, Lref, "fp8", sc=sc) == []
        assert (np.abs(Oe - Oref) <= 0.5 * (U_BF16 * np.abs(Oref) + SIGMAS * sig)).all()
        # scores through the grouped truncation: within the fp8 allowance
        qc, kc = (oracle.e4m3fn_decode(t.view(torch.uint8).numpy()) for t in (q8, k8))
        S = _fp8_scores_truncated(qc[0, hq], kc[0, 0]) * (w.scale * float(desc[0]) * float(desc[1]))
        m = S.max(axis=1)
        P = np.exp(S - m[:, None])
        Ot = round_bf16((round_bf16(P) @ v[0, 0]) / P.sum(axis=1)[:, None])
        Lt = m + np.log(P.sum(axis=1))
        sc8 = scales_head(q[0, hq], k[0, 0], v[0, 0], w.scale, False, rows, Oref, Lref,
                          (qc[0, hq], kc[0, 0], desc[0], desc[1]))
        assert bar_violations(Ot, Lt, Oref, Lref, "fp8", sc=sc8) == []
