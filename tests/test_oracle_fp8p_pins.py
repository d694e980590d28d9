"""Pins for the oracle's e4m3-probability attention (``oracle/fp8p.py``):
per-64-key-block power-of-two scales with exact or Lean P codes.

Each ``check_*`` returns True when the oracle agrees with a fact that does not
come from the module itself:
  * scores whose scaled values are integers in [-6, 8] make every
    probability an exact e4m3 value: both variants equal exact attention;
  * one row worked by hand with torch's e4m3 cast (exact codes) and with an
    e4m3 decoder written here (Lean codes);
  * the block exponent: a block of keys far below another keeps its mass
    (it would be flushed to zero by one scale per row), and a key far below
    the maximum of its own block is flushed;
  * the error statistics the ZYFA article documents: the exact variant is
    within e4m3 precision of exact attention, and Lean P's error is 1-2x the
    exact variant's (the article: 1.22-1.36x).
``test_fp8p_planted_mistakes_are_caught`` plants mistakes in the module.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import oracle.fp8p as ofp
from exact_io_aware_attn_amd.inputs import Workload, make_inputs

LOG2E = 1.4426950408889634


def decode_e4m3(code):
    """OCP e4m3fn value of an integer code 0..126 (positive), written out."""
    e, m = code >> 3, code & 7
    return m * 2.0 ** -9 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7)


def one_row(x, v):
    """One query row with base-2 scores x (1-D) against values v (N, Dv):
    q = [1], k = x, scale = 1 / log2(e) makes the oracle's x_ij equal x."""
    q = np.ones((1, 1))
    k = np.asarray(x, dtype=np.float64)[:, None]
    return q, k, np.asarray(v, dtype=np.float64), 1.0 / LOG2E


def check_integer_scores_are_exact():
    ok = True
    rng = np.random.default_rng(0)
    for trial in range(4):
        N = 150
        # integer base-2 scores within 14 binades of each block's maximum
        x = rng.integers(-5, 9, size=N).astype(np.float64)
        v = rng.standard_normal((N, 3))
        q, k, vv, sc = one_row(x, v)
        Oref, Lref = oracle.attention_head(q, k, vv, sc)
        for lean in (False, True):
            O, L = ofp.fp8p_attention_head(q, k, vv, sc, lean=lean)
            ok &= np.allclose(O, Oref, rtol=0, atol=1e-12) and abs(L[0] - Lref[0]) <= 1e-12
    return ok


def check_hand_worked_row():
    rng = np.random.default_rng(1)
    N = 100
    x = rng.uniform(-9.0, 3.0, size=N)
    x[5] = 3.95    # block maxima with a large fractional part: 2^7.95 fits,
    x[70] = 2.9    # 2^8.95 would not (e4m3 saturates at 448)
    v = rng.standard_normal((N, 2))
    q, k, vv, sc = one_row(x, v)
    ok = True
    for lean in (False, True):
        num, den = np.zeros(2), 0.0
        for b0 in range(0, N, 64):
            xs = x[b0:b0 + 64]
            E = math.ceil(xs.max()) - 8
            for j, xj in enumerate(xs):
                y = xj - E
                if lean:
                    c = int(min(max(np.rint(8 * y + 56), 0), 126))
                    w = decode_e4m3(c)
                else:
                    w = float(torch.tensor([2.0 ** y], dtype=torch.float64).to(torch.float8_e4m3fn).double()[0])
                num += w * 2.0 ** E * v[b0 + j]
                den += w * 2.0 ** E
        O, L = ofp.fp8p_attention_head(q, k, vv, sc, lean=lean)
        ok &= np.allclose(O[0], num / den, rtol=1e-12, atol=1e-12) and abs(L[0] - math.log(den)) <= 1e-12
    return ok


def check_block_exponents():
    ok = True
    v = np.ones((128, 1))
    # key 0 at 0, keys 64..127 at -20: the second block keeps its mass
    x = np.full(128, -1e9)
    x[0] = 0.0
    x[64:] = -20.0
    q, k, vv, sc = one_row(x, v)
    for lean in (False, True):
        _, L = ofp.fp8p_attention_head(q, k, vv, sc, lean=lean)
        ok &= abs(L[0] - math.log(1 + 64 * 2.0 ** -20)) <= 1e-12
    # key 0 at 0 and key 40 at -20 share block 0: key 40 is flushed
    x = np.full(64, -1e9)
    x[0] = 0.0
    x[40] = -20.0
    q, k, vv, sc = one_row(x, np.ones((64, 1)))
    for lean in (False, True):
        _, L = ofp.fp8p_attention_head(q, k, vv, sc, lean=lean)
        ok &= L[0] == 0.0
    return ok


def check_error_statistics():
    ok = True
    for causal in (False, True):
        w = Workload("pin", 1, 2, 2, 256, 256, 128, causal, "fp8", seed=5)
        q8, k8, v8, desc = make_inputs(w)
        x = [oracle.e4m3fn_decode(t.view(torch.uint8).numpy()) * np.float64(d) for t, d in zip((q8, k8, v8), desc)]
        ref, _ = oracle.attention(*x, scale=w.scale, causal=causal)
        rms = lambda o: float(np.sqrt(((o - ref) ** 2).mean()))
        oe, _ = ofp.fp8p_attention(*x, scale=w.scale, causal=causal)
        ol, _ = ofp.fp8p_attention(*x, scale=w.scale, causal=causal, lean=True)
        scale_v = float(np.sqrt((ref ** 2).mean()))
        ok &= rms(oe) <= 2.0 ** -4 * scale_v and 1.0 <= rms(ol) / rms(oe) <= 2.0
    return ok


def check_f32_decisions():
    """The float32-decision form agrees with the float64 form where float32
    rounding is exact (integer scores, c = 1), and with a float32 hand
    computation of one row otherwise."""
    ok = True
    rng = np.random.default_rng(2)
    x = rng.integers(-5, 9, size=150).astype(np.float64)
    v = rng.standard_normal((150, 3))
    q, k, vv, _ = one_row(x, v)
    for lean in (False, True):
        O64, L64 = ofp.fp8p_attention_head(q, k, vv, 1.0 / LOG2E, lean=lean)
        O32, L32 = ofp.fp8p_attention_head_f32(q, k, vv, 1.0, lean=lean)
        ok &= np.allclose(O64, O32, rtol=0, atol=1e-12) and abs(L64[0] - L32[0]) <= 1e-12
    # one row by hand in float32: scores s, multiplier c
    s = rng.integers(-300, 300, size=70).astype(np.float64) / 16.0
    c = np.float32(0.0912)
    q, k, vv, _ = one_row(s, rng.standard_normal((70, 2)))
    for lean in (False, True):
        num, den = np.zeros(2), 0.0
        for b0 in range(0, 70, 64):
            sb = s[b0:b0 + 64]
            E = math.ceil(float(np.float32(np.float32(sb.max()) * c))) - 8
            for j, sj in enumerate(sb):
                if lean:
                    y = np.float32(np.float64(sj) * np.float64(np.float32(8 * c)) + (56.0 - 8 * E))
                    cde = int(min(max(np.rint(y), 0), 126))
                    wgt = decode_e4m3(cde)
                else:
                    y = np.float32(np.float64(sj) * np.float64(c) - E)
                    wgt = float(torch.tensor([2.0 ** float(y)], dtype=torch.float64).to(torch.float8_e4m3fn).double()[0])
                num += wgt * 2.0 ** E * vv[b0 + j]
                den += wgt * 2.0 ** E
        O, L = ofp.fp8p_attention_head_f32(q, k, vv, c, lean=lean)
        ok &= np.allclose(O[0], num / den, rtol=1e-12, atol=1e-12) and abs(L[0] - math.log(den)) <= 1e-12
    return ok


ALL_CHECKS = [check_integer_scores_are_exact, check_hand_worked_row, check_block_exponents, check_error_statistics,
              check_f32_decisions]


@pytest.mark.parametrize("check", ALL_CHECKS, ids=lambda c: c.__name__)
def test_fp8p_oracle_pin(check):
    assert check()


_orig_exponents = ofp.block_exponents
_orig_weights = ofp.fp8p_weights


def _mut_block32(x, vis, block=ofp.BLOCK):
    return _orig_exponents(x, vis, 32)


def _mut_floor(x, vis, block=ofp.BLOCK):
    E = _orig_exponents(x, vis, block)
    R, N = x.shape
    out = E.copy()
    for b in range(E.shape[1]):
        xs = np.where(vis[:, b * block:(b + 1) * block], x[:, b * block:(b + 1) * block], -np.inf)
        mx = xs.max(axis=1)
        out[:, b] = np.where(np.isfinite(mx), np.floor(mx) - ofp.TOP, np.inf)
    return out


def _mut_lean_bias(y):
    return np.clip(np.rint(8.0 * y + 48), 0, 126).astype(np.uint8)


def _mut_lean_trunc(y):
    return np.clip(np.floor(8.0 * y + 56), 0, 126).astype(np.uint8)


def _mut_per_block_norm(x, vis, lean=False, block=ofp.BLOCK):
    w, Ej = _orig_weights(x, vis, lean, block)
    return w, np.zeros_like(Ej)


MUTATIONS = {
    "block_32": (ofp, "block_exponents", _mut_block32),
    "floor_not_ceil": (ofp, "block_exponents", _mut_floor),
    "lean_bias_48": (ofp, "lean_codes", _mut_lean_bias),
    "lean_truncates": (ofp, "lean_codes", _mut_lean_trunc),
    "block_scale_dropped": (ofp, "fp8p_weights", _mut_per_block_norm),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_fp8p_planted_mistakes_are_caught(name, monkeypatch):
    mod, attr, fn = MUTATIONS[name]
    monkeypatch.setattr(mod, attr, fn)
    failed = [c.__name__ for c in ALL_CHECKS if not c()]
    assert failed, f"no check caught the planted mistake {name}"


def test_poly_exp2_error_bound():
    """The cubic meets its stated bound against numpy's exp2 (relative error
    at most 8.6e-5 over a dense grid of [-126, 8]), is exact at integers
    (f = 0), and underflows to 0 at -150 and below, -inf included."""
    y = np.linspace(-126.0, 8.0, 2_000_001)
    rel = np.abs(oracle.poly_exp2(y) / np.exp2(y) - 1.0)
    assert rel.max() <= 8.6e-5
    ints = np.arange(-126, 9, dtype=np.float64)
    assert np.array_equal(oracle.poly_exp2(ints), np.exp2(ints))
    assert oracle.poly_exp2(np.array([-250.0, -np.inf])).tolist() == [0.0, 0.0]


def test_poly_exp2_planted_mistake_is_caught(monkeypatch):
    """A coefficient slip (b and c swapped) breaks the bound."""
    import oracle.polyexp as ope
    monkeypatch.setattr(ope, "COEFFS", (ope.COEFFS[0], ope.COEFFS[2], ope.COEFFS[1]))
    y = np.linspace(-10.0, 8.0, 100_001)
    assert np.abs(ope.poly_exp2(y) / np.exp2(y) - 1.0).max() > 8.6e-5
