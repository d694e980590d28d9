"""Attention with e4m3 probabilities: one power-of-two scale per 64-key block
of each row, exact or "Lean P" codes.  float64 on the CPU.

TEST INFRASTRUCTURE ONLY (see the package docstring).

ZYFA article, section "The three techniques, in plain terms":
  * Per-block scaling with a rounded row sum: most probabilities lie many
    binades below the row maximum, where e4m3 values are subnormal or zero;
    each 64-key block of probabilities is multiplied by a power of two before
    rounding, the P V product divides it back out, and the denominator is
    the sum of the same rounded probabilities, so the output is a true
    weighted average whose weights sum to one.
  * Lean P: read as an integer, the code of a positive e4m3 number grows by 8
    per doubling, so the code is about 8 log2(value) plus a constant; a
    probability 2^(score - max) gets its code from one multiply-add and an
    integer conversion instead of an exponential and a conversion.  Its error
    is documented as 1.22-1.36x that of the exact version.

What is computed, for one row i (readings where the article is silent):
  x_ij  = scale * log2(e) * q_i . k_j          (base-2 scores)
  blocks: keys [64 b, 64 b + 64) of the key sequence; only visible keys count
  E_ib  = ceil(max over visible j in block b of x_ij) - 8
          (the largest scaled value of a block falls in (2^7, 2^8])
  exact:  code_ij = e4m3fn(2^(x_ij - E_ib))     nearest, ties to even
  lean:   code_ij = clamp(rne(8 (x_ij - E_ib) + 56), 0, 126) as an integer
          (exact wherever x_ij - E_ib is an integer in [-6, 8]: the code of
          2^e is 8 (e + 7); between, the mantissa runs linearly in the
          fraction, the linear reading of the article's "8 times the base-2
          logarithm plus a constant")
  p_ij  = decode(code_ij) * 2^E_ib              (0 for invisible keys)
  O_i   = sum_j p_ij v_j / sum_j p_ij,   LSE_i = ln(sum_j p_ij)
A row that sees no key has O = 0, LSE = -inf.  p_ij approximates
exp(scale q_i . k_j) itself, so no running maximum appears in the result.

``fp8p_attention_head_f32`` takes the same rounding decisions (block
exponent, code) from float32 values computed as the device computes them
(one rounding after each multiply-add), for parity at the level of
individual codes; its inputs must keep q . k exact in float32.
"""
import numpy as np

from .e4m3 import e4m3fn_decode
from .exact import kv_head_of, visible_mask
from .quant import e4m3fn_encode

LOG2E = 1.4426950408889634
BLOCK = 64
TOP = 8           # the block maximum maps into (2^(TOP-1), 2^TOP]
LEAN_BIAS = 56    # e4m3 code of 2^e is 8 (e + 7): 8 log2(v) + 56


def block_exponents(x, vis, block=BLOCK):
    """E (rows, n_blocks): ceil of each block's largest visible score minus
    TOP; +inf where a block has no visible key."""
    R, N = x.shape
    nb = (N + block - 1) // block
    E = np.full((R, nb), np.inf)
    for b in range(nb):
        xs = np.where(vis[:, b * block:(b + 1) * block], x[:, b * block:(b + 1) * block], -np.inf)
        mx = xs.max(axis=1)
        E[:, b] = np.where(np.isfinite(mx), np.ceil(mx) - TOP, np.inf)
    return E


def lean_codes(y):
    """Lean P codes of scaled base-2 values y = x - E: rne(8 y + 56) clamped
    to [0, 126]."""
    return np.clip(np.rint(8.0 * y + LEAN_BIAS), 0, 126).astype(np.uint8)


def fp8p_weights(x, vis, lean=False, block=BLOCK):
    """The weights p_ij of the rows of base-2 scores x (rows, N) with
    visibility vis, as (mantissa part, exponent part): p = w * 2^E."""
    E = block_exponents(x, vis, block)
    Ej = np.repeat(E, block, axis=1)[:, : x.shape[1]]
    y = np.where(vis, x - np.where(np.isfinite(Ej), Ej, 0.0), -np.inf)
    if lean:
        codes = np.where(vis, lean_codes(np.where(vis, y, 0.0)), 0).astype(np.uint8)
    else:
        codes = np.where(vis, e4m3fn_encode(np.where(vis, np.exp2(y), 0.0)), 0).astype(np.uint8)
    w = np.where(vis, e4m3fn_decode(codes), 0.0)
    return w, np.where(vis, Ej, 0.0)


def fp8p_attention_head(q, k, v, scale, causal=False, lean=False, rows=None, block=BLOCK):
    """O (len(rows), Dv) and natural-log LSE for one (batch, query head)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    Nq, Nkv = q.shape[0], k.shape[0]
    if rows is None:
        rows = np.arange(Nq)
    rows = np.asarray(rows, dtype=np.int64)
    vis = visible_mask(Nq, Nkv, causal, rows)
    x = (q[rows] @ k.T) * (np.float64(scale) * LOG2E)
    w, Ej = fp8p_weights(x, vis, lean, block)
    any_vis = vis.any(axis=1)
    # weights relative to each row's largest exponent (range safety)
    Emax = np.where(any_vis, np.where(vis, Ej, -np.inf).max(axis=1), 0.0)
    p = w * np.exp2(np.where(vis, Ej - Emax[:, None], 0.0))
    l = p.sum(axis=1)
    O = np.where(any_vis[:, None] & (l[:, None] > 0), (p @ v) / np.where(l > 0, l, 1.0)[:, None], 0.0)
    lse = np.where(any_vis & (l > 0), (np.log2(np.where(l > 0, l, 1.0)) + Emax) / LOG2E, -np.inf)
    return O, lse


def fp8p_attention(q, k, v, scale, causal=False, lean=False):
    """Whole (B, H, N, D) problem; returns O, LSE (float64)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, Hq, Nq, _ = q.shape
    Hkv = k.shape[1]
    O = np.empty(q.shape[:3] + (v.shape[3],), dtype=np.float64)
    lse = np.empty((B, Hq, Nq), dtype=np.float64)
    for b in range(B):
        for hq in range(Hq):
            hk = kv_head_of(hq, Hq, Hkv)
            O[b, hq], lse[b, hq] = fp8p_attention_head(q[b, hq], k[b, hk], v[b, hk], scale, causal, lean)
    return O, lse


def _f32(x):
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def fp8p_attention_head_f32(q, k, v, c32, causal=False, lean=False, rows=None, block=BLOCK):
    """The weights of ``fp8p_attention_head`` with every rounding decision
    taken in float32, as the device takes it:
      s_ij  = q_i . k_j (q, k the e4m3 values without descales; the caller
              keeps these sums exact in float32),
      c32   = the float32 multiplier scale * log2(e) * dq * dk,
      E     = ceil(f32(max_j s_ij * c32)) - 8 per 64-key block,
      exact: code = e4m3(2^f32(s_ij c32 - E))  (one rounding: a multiply-add)
      lean:  code = rne(f32(s_ij f32(8 c32) + f32(56 - 8 E))), clamped to [0, 126]
    and O, LSE as ``fp8p_attention_head`` (v carries its descale)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    c32 = float(np.float32(c32))
    Nq, Nkv = q.shape[0], k.shape[0]
    if rows is None:
        rows = np.arange(Nq)
    rows = np.asarray(rows, dtype=np.int64)
    vis = visible_mask(Nq, Nkv, causal, rows)
    S = q[rows] @ k.T                                   # exact by the caller's choice of inputs
    R, N = S.shape
    nb = (N + block - 1) // block
    w = np.zeros((R, N))
    Ej = np.zeros((R, N))
    for b in range(nb):
        sl = slice(b * block, min((b + 1) * block, N))
        vb = vis[:, sl]
        smax = np.where(vb, S[:, sl], -np.inf).max(axis=1)
        has = np.isfinite(smax)
        E = np.where(has, np.ceil(_f32(np.where(has, smax, 0.0) * c32)) - TOP, 0.0)
        if lean:
            c8 = float(np.float32(8.0 * c32))
            y = _f32(S[:, sl] * c8 + _f32(LEAN_BIAS - 8.0 * E)[:, None])
            codes = np.clip(np.rint(y), 0, 126).astype(np.uint8)
        else:
            y = _f32(S[:, sl] * c32 - E[:, None])
            codes = e4m3fn_encode(np.exp2(y))
        w[:, sl] = np.where(vb, e4m3fn_decode(codes), 0.0)
        Ej[:, sl] = E[:, None]
    any_vis = vis.any(axis=1)
    Emax = np.where(any_vis, np.where(vis, Ej, -np.inf).max(axis=1), 0.0)
    p = w * np.exp2(np.where(vis, Ej - Emax[:, None], 0.0))
    l = p.sum(axis=1)
    O = np.where(any_vis[:, None] & (l[:, None] > 0), (p @ v) / np.where(l > 0, l, 1.0)[:, None], 0.0)
    lse = np.where(any_vis & (l > 0), (np.log2(np.where(l > 0, l, 1.0)) + Emax) / LOG2E, -np.inf)
    return O, lse
