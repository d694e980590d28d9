"""CPU pins of the boundary-aware bounds (``fp8_bounds.py``) that the GPU
tests of the rotated quantiser and of e4m3-probability attention apply.

Each bound must (a) admit the outcomes of a float32 computation that decides
like the device (so a correct device passes), (b) reject a planted mistake
away from a decision boundary (so the GPU check is not vacuous), and
(c) flag only a small fraction of decisions as ambiguous.
"""
import numpy as np
import pytest
import torch

import oracle
from exact_io_aware_attn_amd.inputs import Workload, make_inputs
from fp8_bounds import fp8p_row_bounds, ordinal, rotated_code_intervals


def _fwht_f32(x, signs):
    """The rotation in float32 butterflies (a different order from the
    device's, within the same error bound): signs, log2(D) add/sub stages,
    then the float32 multiply by 1 / sqrt(D)."""
    y = (x * signs).astype(np.float32)
    D = y.shape[-1]
    h = 1
    while h < D:
        y = y.reshape(*y.shape[:-1], D // (2 * h), 2, h)
        a, b = y[..., 0, :].copy(), y[..., 1, :].copy()
        y[..., 0, :] = a + b
        y[..., 1, :] = a - b
        y = y.reshape(*y.shape[:-3], D)
        h *= 2
    return (y * np.float32(1.0 / np.sqrt(D))).astype(np.float32)


def _quantize_f32(xr32, block=64):
    """Block quantisation of already rotated float32 values, float32
    decisions (amax, 448 / amax, the product), nearest e4m3 code."""
    B, H, N, D = xr32.shape
    codes = np.empty(xr32.shape, dtype=np.uint8)
    for i in range(0, N, block):
        blk = xr32[:, :, i:i + block]
        amax = np.abs(blk).max(axis=(2, 3)).astype(np.float32)
        inv = np.where(amax == 0, np.float32(0), np.float32(448.0) / np.where(amax == 0, np.float32(1), amax))
        y = np.clip((blk * inv.astype(np.float32)[:, :, None, None]).astype(np.float32), -448, 448)
        codes[:, :, i:i + block] = oracle.e4m3fn_encode(y)
    return codes


@pytest.mark.parametrize("D", [64, 128, 256])
def test_rotated_code_intervals(D):
    w = Workload("fp8blk", 2, 3, 3, 300, 300, D, False, "fp8blk", outlier_frac=0.01, seed=D)
    q, _, _, signs = make_inputs(w)
    x = q.to(torch.float64).numpy()
    x[:, :, 64:128] = 0.0          # a block of zeros (descale 1, codes 0)
    x[0, 0, 64, 0] = -0.0
    s = signs.numpy().astype(np.float64)
    lo, hi, dlo, dhi = rotated_code_intervals(x, s)
    # (a) the oracle's decisions and a float32 rotation's decisions lie inside
    c_ref, d_ref = oracle.quantize_blocks(x, s)
    assert ((lo <= ordinal(c_ref)) & (ordinal(c_ref) <= hi)).all()
    assert ((dlo <= d_ref) & (d_ref <= dhi)).all()
    c32 = _quantize_f32(_fwht_f32(x, s))
    o32 = ordinal(c32)
    assert ((lo <= o32) & (o32 <= hi)).all()
    # (c) few decisions are ambiguous, and those are where the two differ
    amb = lo != hi
    assert amb.mean() < 5e-3, amb.mean()
    assert ((o32 == ordinal(c_ref)) | amb).all()
    # (b) one code a step off where the decision is not ambiguous is caught
    idx = tuple(np.argwhere(~amb & (np.abs(ordinal(c_ref)) > 8))[7])
    bad = ordinal(c_ref).copy()
    bad[idx] += 1
    assert not ((lo <= bad) & (bad <= hi)).all()


def _codes(w):
    q8, k8, v8, desc = make_inputs(w)
    qc, kc, vc = (oracle.e4m3fn_decode(t.view(torch.uint8).numpy()) for t in (q8, k8, v8))
    return qc, kc, vc * np.float64(desc[2]), desc


@pytest.mark.parametrize("lean", [False, True], ids=["exact", "lean"])
def test_fp8p_bounds_admit_float32_decisions(lean):
    """The oracle's float32-decision variant (scores rounded once to float32
    as the device's multiply-add rounds them) is an admissible device."""
    w = Workload("p8b", 1, 2, 2, 300, 700, 128, True, "fp8", seed=9, outlier_frac=0.01)
    qc, kc, v, desc = _codes(w)
    c32 = np.float32(np.float32(np.float32(w.scale) * np.float32(1.4426950408889634)) * desc[0]) * desc[1]
    rows = np.arange(w.Nq)
    n_amb = 0
    for h in range(w.Hq):
        O, L, bO, bL, amb, _ = fp8p_row_bounds(qc[0, h], kc[0, h], v[0, h], desc[0], desc[1], w.scale, True, lean,
                                               rows)
        n_amb += int(amb.sum())
        # same weights as the plain float64 oracle
        O64, L64 = oracle.fp8p_attention_head(qc[0, h] * np.float64(desc[0]), kc[0, h] * np.float64(desc[1]),
                                              v[0, h], w.scale, True, lean=lean)
        assert np.allclose(O, O64, rtol=1e-12, atol=1e-12) and np.allclose(L, L64, rtol=1e-12, atol=1e-12)
        Of, Lf = oracle.fp8p_attention_head_f32(qc[0, h], kc[0, h], v[0, h], c32, True, lean=lean)
        assert (np.abs(Of - O) <= bO + 1e-9).all()
        fin = np.isfinite(L)
        assert (np.abs(Lf[fin] - L[fin]) <= bL[fin] + 1e-9).all()
    # the fp8 matrix instruction's grouped accumulation leaves a few per cent
    # of the decisions on these outlier inputs open
    assert 0 < n_amb < 0.05 * w.Hq * w.visible_pairs


@pytest.mark.parametrize("lean", [False, True], ids=["exact", "lean"])
def test_fp8p_bounds_reject_planted_mistakes(lean):
    """A code one step off at a row's largest weight whose decision is not
    open moves O or LSE beyond the admissible deviation in every row; a dropped 64-key block (1/32 of
    the keys) in nine rows of ten."""
    w = Workload("p8m", 1, 1, 1, 2048, 2048, 128, False, "fp8", seed=0, outlier_frac=0.01)
    qc, kc, v, desc = _codes(w)
    rows = np.arange(0, w.Nq, 97)
    O, L, bO, bL, amb, _ = fp8p_row_bounds(qc[0, 0], kc[0, 0], v[0, 0], desc[0], desc[1], w.scale, False, lean, rows)
    x = (qc[0, 0][rows] @ kc[0, 0].T) * (w.scale * 1.4426950408889634 * float(desc[0]) * float(desc[1]))
    vis = np.ones_like(x, dtype=bool)
    wts, Ej = oracle.fp8p.fp8p_weights(x, vis, lean)
    p = wts * np.exp2(Ej)
    caught = dropped = 0
    for i in range(rows.size):
        j = int(np.argmax(np.where(amb[i], -1.0, p[i])))   # the largest weight with a settled code
        code = oracle.e4m3fn_encode(wts[i, j])
        p2 = p[i].copy()
        p2[j] = oracle.e4m3fn_decode(np.uint8(int(code) + 1)) * np.exp2(Ej[i, j])
        O2 = (p2 @ v[0, 0]) / p2.sum()
        L2 = np.log(p2.sum())
        caught += bool((np.abs(O2 - O[i]) > bO[i]).any() or abs(L2 - L[i]) > bL[i])
        # a dropped block of 64 keys: beyond the output bound or the LSE
        # bound plus the 5e-4 bar
        keep = np.ones(w.Nkv, dtype=bool)
        keep[1024:1088] = False
        O3 = (p[i][keep] @ v[0, 0][keep]) / p[i][keep].sum()
        L3 = np.log(p[i][keep].sum())
        dropped += bool((np.abs(O3 - O[i]) > bO[i]).any() or abs(L3 - L[i]) > bL[i] + 5e-4)
    # a row whose weight sits on a key with an open code decision admits a
    # deviation of one code step there (1/8 of that weight), which can
    # exceed a low-weight block; all other rows see the dropped block
    assert caught == rows.size and dropped >= 0.9 * rows.size
