"""Boundary-aware parity for results decided by rounding: which device
outcomes are admissible given the float32 arithmetic the device decides in.

Where a byte or an integer is decided from a floating-point value, the
device (float32) and the oracle (float64) may decide differently only where
the oracle's float64 decision input lies within the float32 arithmetic's
error bound of a decision boundary.  These helpers compute, from the
oracle's float64 values and rigorous float32 error bounds, the set of
outcomes the device may produce; the GPU tests then require the device's
outcome to lie in that set, element by element, so a mismatch anywhere
else fails.

* ``rotated_code_intervals``: the rotated block quantiser (e4m3 codes of x R
  times 448 / amax).  Bound of the device's fast Walsh-Hadamard transform:
  log2(D) butterfly stages, each an fp32 add with one rounding, so the
  rotated value is off by at most log2(D) u sum_j |x_j| / sqrt(D), plus two
  roundings of the normalisation; the block amax, 448 / amax and the
  product follow, each with its own rounding.
* ``fp8p_row_bounds``: attention with e4m3 probabilities (exact or Lean P
  codes, one power-of-two scale per 64-key block).  Bound on the device's
  base-2 scores: the fp8 matrix instruction's grouped accumulation of the
  D products (``bars.fp8_dot_error_bound``); the fp32 multiplier scale *
  log2(e) * dq * dk carries five roundings and the multiply-add one more.
  Each block exponent and each code may take any value reachable within
  that bound; the admissible deviation of each weight bounds the deviation
  of the row's output and LSE.  ``fp8p_accumulation_bound`` adds the same
  instruction's grouped accumulation in P V and in the row sum.

u = 2^-24 throughout (float32 unit roundoff).
"""
import math

import numpy as np

import oracle
from bars import fp8_dot_error_bound, fp8_group_error
from oracle.fp8p import BLOCK, LEAN_BIAS, LOG2E, TOP, lean_codes

U32 = 2.0 ** -24
EXP2_REL = 2.0 ** -22   # v_exp_f32: within 1 ulp of 2^x (2 ulps taken)


def ordinal(codes):
    """Signed position of an e4m3fn code on the number line (+-0 both 0)."""
    c = np.asarray(codes).astype(np.int64)
    m = c & 0x7F
    return np.where(c & 0x80, -m, m)


def rotated_code_intervals(x, signs, block=64):
    """Admissible device outcomes of the rotated block quantiser.

    x: (B, H, N, D) float64 (the bf16 input values), signs: (D,) of +-1.
    Returns (code_lo, code_hi, d_lo, d_hi): the ordinal range each code may
    take (ordinal() of the device codes must lie in it) and the range of
    each block's descale, (B, H, ceil(N / block))."""
    x = np.asarray(x, dtype=np.float64)
    B, H, N, D = x.shape
    L = int(math.log2(D))
    xr = x @ oracle.rotation(signs)                          # float64, error ~1e-16
    # device error bound of each rotated value
    s_row = np.abs(x).sum(axis=-1, keepdims=True)
    delta = (L * U32 * s_row / math.sqrt(D)) * (1 + 1e-6) + 2.01 * U32 * np.abs(xr) + 1e-45
    nb = (N + block - 1) // block
    code_lo = np.empty(x.shape, dtype=np.int64)
    code_hi = np.empty(x.shape, dtype=np.int64)
    d_lo = np.empty((B, H, nb))
    d_hi = np.empty((B, H, nb))
    for i in range(nb):
        sl = slice(i * block, min((i + 1) * block, N))
        a, dl = np.abs(xr[:, :, sl]), delta[:, :, sl]
        # a block of zero inputs rotates to exact zeros: descale 1, codes 0
        zero = (x[:, :, sl] == 0).all(axis=(2, 3))
        amax_lo = np.maximum(a - dl, 0.0).max(axis=(2, 3))
        amax_hi = (a + dl).max(axis=(2, 3))
        d_lo[:, :, i] = np.where(zero, 1.0, amax_lo / 448.0 * (1 - U32))
        d_hi[:, :, i] = np.where(zero, 1.0, amax_hi / 448.0 * (1 + U32))
        inv_lo = np.where(zero, 0.0, 448.0 / np.where(zero, 1.0, amax_hi) * (1 - U32))
        inv_hi = np.where(zero | (amax_lo == 0), np.inf, 448.0 / np.where(amax_lo == 0, 1.0, amax_lo) * (1 + U32))
        inv_lo, inv_hi = inv_lo[:, :, None, None], inv_hi[:, :, None, None]
        xlo, xhi = xr[:, :, sl] - dl, xr[:, :, sl] + dl
        with np.errstate(invalid="ignore"):
            cands = np.stack([xlo * inv_lo, xlo * inv_hi, xhi * inv_lo, xhi * inv_hi])
        cands = np.where(np.isnan(cands), 0.0, cands)     # 0 * inf: a zero block
        ylo = cands.min(axis=0)
        yhi = cands.max(axis=0)
        ylo = np.clip(ylo - U32 * np.abs(ylo), -448.0, 448.0)
        yhi = np.clip(yhi + U32 * np.abs(yhi), -448.0, 448.0)
        zb = zero[:, :, None, None]
        ylo = np.where(zb, 0.0, ylo)
        yhi = np.where(zb, 0.0, yhi)
        code_lo[:, :, sl] = ordinal(oracle.e4m3fn_encode(ylo))
        code_hi[:, :, sl] = ordinal(oracle.e4m3fn_encode(yhi))
    return code_lo, code_hi, d_lo, d_hi


def _codes(y, lean):
    """Codes of the scaled base-2 values y (visible entries)."""
    if lean:
        return lean_codes(y)
    return oracle.e4m3fn_encode(np.exp2(y))


def fp8p_row_bounds(qc, kc, v, dq, dk, scale, causal, lean, rows, block=BLOCK):
    """Oracle result and admissible device deviation for rows of one
    (batch, head) of e4m3-probability attention.

    qc, kc: e4m3 code values (decoded, without descales), (Nq, D), (Nkv, D);
    v: the values (decoded codes times dv), (Nkv, Dv); dq, dk: the per-tensor
    descales (float32 values); scale: the softmax scale.
    Returns (O, LSE, bound_O, bound_LSE, ambiguous, p): O and LSE of the
    oracle's float64 decisions, and bounds such that every admissible device
    output satisfies |O_dev - O| <= bound_O (element by element, before
    the device's accumulation in P V and the bf16 rounding of O) and
    |LSE_dev - LSE| <= bound_LSE; p the rows' weights relative to each
    row's largest block exponent (for ``fp8p_accumulation_bound``);
    ambiguous (R, Nkv) marks the weights with more than one admissible
    value."""
    qc = np.asarray(qc, dtype=np.float64)
    kc = np.asarray(kc, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    rows = np.asarray(rows, dtype=np.int64)
    Nq, Nkv = qc.shape[0], kc.shape[0]
    D = qc.shape[1]
    vis = oracle.visible_mask(Nq, Nkv, causal, rows)
    s = qc[rows] @ kc.T                                  # exact in float64 (e4m3 products, D terms)
    c = float(scale) * LOG2E * float(dq) * float(dk)
    x = s * c
    # device score error: the matrix instruction's grouped accumulation, the
    # multiplier's five roundings and the multiply-add's one
    dx = abs(c) * fp8_dot_error_bound(qc[rows], kc) * (1 + 1e-6) + 7 * U32 * np.abs(x) + 1e-30
    w, Ej = oracle.fp8p.fp8p_weights(x, vis, lean, block)
    p = w * np.exp2(Ej)
    R = rows.size
    nb = (Nkv + block - 1) // block
    pmin = p.copy()
    pmax = p.copy()
    n_amb = 0
    for b in range(nb):
        sl = slice(b * block, min((b + 1) * block, Nkv))
        vb = vis[:, sl]
        has = vb.any(axis=1)
        if not has.any():
            continue
        xb = np.where(vb, x[:, sl], -np.inf)
        mx = xb.max(axis=1)
        dm = np.where(vb, dx[:, sl], 0.0).max(axis=1) + U32 * np.abs(np.where(has, mx, 0.0))
        e_lo = np.where(has, np.ceil(np.where(has, mx, 0.0) - dm) - TOP, 0.0)
        e_hi = np.where(has, np.ceil(np.where(has, mx, 0.0) + dm) - TOP, 0.0)
        for E in np.unique(np.concatenate([e_lo[has], e_hi[has]])):
            rows_e = has & (e_lo <= E) & (E <= e_hi)
            if not rows_e.any():
                continue
            Ec = np.full(R, E)[:, None]
            y = x[:, sl] - Ec
            dy = dx[:, sl] + U32 * (np.abs(y) + abs(E))
            if lean:
                t = 8.0 * y + LEAN_BIAS
                dt = 8.0 * dy + U32 * np.abs(t)
                lo = _codes((t - dt - LEAN_BIAS) / 8.0, True)
                hi = _codes((t + dt - LEAN_BIAS) / 8.0, True)
            else:
                lo = oracle.e4m3fn_encode(np.exp2(y - dy) * (1 - EXP2_REL))
                hi = oracle.e4m3fn_encode(np.exp2(y + dy) * (1 + EXP2_REL))
            plo = oracle.e4m3fn_decode(lo) * np.exp2(E)
            phi = oracle.e4m3fn_decode(hi) * np.exp2(E)
            sel = vb & rows_e[:, None]
            pmin[:, sl] = np.where(sel, np.minimum(pmin[:, sl], plo), pmin[:, sl])
            pmax[:, sl] = np.where(sel, np.maximum(pmax[:, sl], phi), pmax[:, sl])
    dev = np.where(vis, np.maximum(p - pmin, pmax - p), 0.0)
    n_amb = int((dev > 0).sum())
    # oracle output and LSE on the float64 decisions, weights relative to
    # each row's largest exponent (as the oracle forms them)
    any_vis = vis.any(axis=1)
    Emax = np.where(any_vis, np.where(vis, Ej, -np.inf).max(axis=1), 0.0)
    f = np.exp2(-Emax)[:, None]
    pr, devr = p * f, dev * f
    l = pr.sum(axis=1)
    ok = any_vis & (l > 0)
    ls = np.where(ok, l, 1.0)
    O = np.where(ok[:, None], (pr @ v) / ls[:, None], 0.0)
    LSE = np.where(ok, (np.log2(ls) + Emax) / LOG2E, -np.inf)
    dsum = devr.sum(axis=1)
    den = np.maximum(ls - dsum, 1e-300)
    # |O' - O| <= sum_j dev_j |v_j - O| / (l - sum_j dev_j)
    bO = np.empty_like(O)
    for i in range(R):
        bO[i] = (devr[i] @ np.abs(v - O[i][None, :])) / den[i] if ok[i] else 0.0
    bL = np.where(ok, np.log(ls / den), 0.0)
    return O, LSE, bO, bL, dev > 0, pr


def _pv_groups(n):
    """Key groups of the P V instruction's grouped accumulation in the
    e4m3-probability kernel: the 8 consecutive bytes of a lane's P operand
    hold keys 32 kb + 4 h + {0..3, 8..11} (+ 16 for the second 8 bytes) of
    a 64-key tile, kb and h the key block and lane half.  Returns (G, 8)
    key indices, keys past n pointing at n (a zero pad)."""
    tiles = (n + 63) // 64
    groups = []
    for t in range(tiles):
        for kb in range(2):
            for rh in range(2):
                for h in range(2):
                    base = 64 * t + 32 * kb + 16 * rh + 4 * h
                    groups.append([base + i for i in range(4)] + [base + 8 + i for i in range(4)])
    g = np.asarray(groups)
    return np.where(g < n, g, n)


def fp8p_accumulation_bound(O, p, v, block=BLOCK):
    """Bound of the device's accumulation error in P V and in the row sum of
    e4m3-probability attention, for one row: O (Dv,) the row's output, p
    (N,) its weights (relative, as the row sum sees them), v (N, Dv).  The
    fp8 instruction's grouped accumulation (``bars.fp8_group_error``) plus
    one fp32 rounding per 64-key tile: err_N for the numerator, err_l for
    the row sum: returns (|dO| bound (Dv,), |dLSE| bound), |dO| <=
    (err_N + |O| err_l) / (l - err_l) and |dLSE| <= ln(l / (l - err_l))."""
    n = p.shape[0]
    g = _pv_groups(n)
    pz = np.concatenate([p, [0.0]])
    vz = np.concatenate([v, np.zeros((1, v.shape[1]))])
    pg = pz[g]                                               # (G, 8)
    prod = np.abs(pg[:, :, None] * vz[g])                     # (G, 8, Dv)
    tiles = (n + block - 1) // block
    err_n = fp8_group_error(np.moveaxis(prod, 2, 0)) + (tiles + 2) * U32 * prod.sum(axis=(0, 1))
    err_l = fp8_group_error(np.abs(pg)) + (tiles + 2) * U32 * p.sum()
    l = p.sum()
    den = max(l - err_l, 1e-300)
    return (err_n + np.abs(O) * err_l) / den, float(np.log(l / den)) if l > 0 else 0.0
