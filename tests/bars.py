"""Parity bars shared by the GPU parity tests and their CPU sensitivity tests.

Every exact path is held to two kinds of bar:

* the stated tolerances: max |dO| <= 2e-2 (bf16), 8e-2 (fp8), 1e-4 (fp32),
  and |dLSE| <= 1e-3 * max(1, |LSE|);
* scale-aware bars, which a kernel that silently dropped one key tile fails
  at full size, where the outputs are small (|O| of a few 1e-2 over
  thousands of keys, so the absolute 2e-2 bar alone carries no information):
    - |dLSE| <= 5e-4 absolute.  LSE comes from an fp32 running maximum and
      an fp32 sum of the unrounded probabilities (error ~1e-6); dropping 32
      of N keys moves it by about -ln(1 - 32/N) (3.9e-3 at N = 8192).  For
      e4m3 inputs the scores come from the fp8 matrix instruction, whose
      grouped accumulation (``fp8_dot_error_bound`` below) adds the row's
      bound of its score error.
    - element by element, |dO_id| <= 2^-8 |O_id| + 8 sigma_id with
      sigma_id = 2^-8 / sqrt(3) * sqrt(sum_j w_ij^2 v_jd^2), w the exact
      softmax weights.  A correct bf16-P kernel rounds each probability to
      bf16 (relative error within +-2^-8, the unit roundoff of 8
      significant bits, so O_id moves by a sum of independent terms
      w_ij e_j v_jd of standard deviation at most sigma_id) and O to bf16
      (at most 2^-8 |O_id|); 8 sigma bounds the first for every element of
      every test, and is at least the worst case 2^-8 sum_j w_ij |v_jd|
      whenever fewer than 21 keys carry the weight.  Dropping 32 of 4096
      keys moves O by ~sqrt(32) / 4096 |v| per channel, tens of sigma.  For
      e4m3 inputs the score error bound adds its effect on the weights.
  The output bar is relative to the row's own rounding scale, not to max |O|:
  with outlier channels a row's output can be a near cancellation of large
  values, whose rounding error is far above 2^-8 |O|.  It applies where
  probabilities are rounded to bf16 (bf16 and e4m3 inputs); fp32 inputs keep
  fp32 probabilities and the 1e-4 absolute bar.
"""
import numpy as np

import oracle

TOL_O = {"f32": 1e-4, "bf16": 2e-2, "fp8": 8e-2}
TOL_LSE_REL = 1e-3
ABS_LSE = 5e-4
SIGMAS = 8.0
U_BF16 = 2.0 ** -8  # unit roundoff of bf16 (8 significant bits)


U32 = 2.0 ** -24
# The scaled fp8 matrix instruction (v_mfma_scale_f32_32x32x64_f8f6f4) adds
# its products in groups of 8 consecutive contraction indices on a grid of
# 2^(e - 13), e the exponent of the group's largest product (measured on
# gfx950 with a single instruction: 448 plus 63 small terms keeps terms of
# 2^-5 and drops the 7 terms of 2^-6 and below that share the large term's
# group, and only those).  A product of two e4m3 values has at most 8
# significant bits, so products of exponent e - 6 or more lie on that grid
# and are exact; smaller ones lose at most one grid step.  Bound taken, with
# a factor 2 of margin on the grid: per group, the sum over its products
# below 2^(e - 5) of min(|product|, 2^(e - 12)), plus one fp32 rounding of
# each group sum.
FP8_GROUP = 8
FP8_GRID = 12      # grid step 2^(e - FP8_GRID) taken (measured: 13)


def fp8_dot_error_bound(a, b):
    """Bound of |device - exact| for the dot products of the rows of a
    (R, K) with the rows of b (N, K) on the fp8 matrix instruction, groups
    of FP8_GROUP consecutive contraction indices; (R, N)."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    R, K = a.shape
    out = np.empty((R, b.shape[0]))
    ab = np.abs(b).reshape(b.shape[0], K // FP8_GROUP, FP8_GROUP)
    for i in range(R):
        prod = np.abs(a[i]).reshape(1, K // FP8_GROUP, FP8_GROUP) * ab
        mx = prod.max(axis=2, keepdims=True)
        e = np.floor(np.log2(np.where(mx > 0, mx, 1.0)))
        step = np.exp2(e - FP8_GRID)
        lossy = prod < np.exp2(e - FP8_GRID + 7)
        err = np.where(lossy, np.minimum(prod, step), 0.0).sum(axis=2)
        out[i] = err.sum(axis=1) + (K // FP8_GROUP + 2) * U32 * prod.sum(axis=(1, 2))
    return out


def fp8_group_error(prod):
    """The same bound for groups given directly: prod (..., G, 8) absolute
    products; returns the bound summed over G, shape (...)."""
    mx = prod.max(axis=-1, keepdims=True)
    e = np.floor(np.log2(np.where(mx > 0, mx, 1.0)))
    step = np.exp2(e - FP8_GRID)
    lossy = prod < np.exp2(e - FP8_GRID + 7)
    return np.where(lossy, np.minimum(prod, step), 0.0).sum(axis=(-2, -1))


def scales_head(q, k, v, scale, causal, rows, Oref, Lref, fp8=None):
    """Per-row error scales of one (batch, head) for the scale-aware bars.

    sigma_id = 2^-8 / sqrt(3) * sqrt(sum_j w_ij^2 v_jd^2), w the exact
    softmax weights exp(s_ij - LSE_i) (zero for invisible keys and keyless
    rows).  With ``fp8`` = (q codes, k codes, dq, dk) -- e4m3 inputs, whose
    scores come from the fp8 matrix instruction -- also the bound of each
    row's score error e_i = max over visible j of scale dq dk
    fp8_dot_error_bound, and its effect on O, 1.1 e_i sum_j w_ij |v_jd -
    O_id| (weights perturbed by factors within exp(+-e_i)); LSE moves by at
    most e_i."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    rows = np.asarray(rows, dtype=np.int64)
    S = (q[rows] @ k.T) * np.float64(scale)
    vis = oracle.visible_mask(q.shape[0], k.shape[0], causal, rows)
    fin = np.isfinite(Lref)
    w = np.where(vis & fin[:, None], np.exp(np.where(vis, S, 0.0) - np.where(fin, Lref, 0.0)[:, None]), 0.0)
    out = {"sigma": U_BF16 / np.sqrt(3.0) * np.sqrt((w * w) @ (v * v))}
    if fp8 is not None:
        qc, kc, dq, dk = fp8
        eb = fp8_dot_error_bound(np.asarray(qc)[rows], kc) * (abs(float(scale)) * float(dq) * float(dk))
        e = np.where(vis, eb, 0.0).max(axis=1)
        out["lse_extra"] = e
        spread = np.stack([w[i] @ np.abs(v - Oref[i][None, :]) for i in range(rows.size)]) if rows.size else \
            np.zeros((0, v.shape[1]))
        out["o_extra"] = 1.1 * e[:, None] * spread
    return out


def scales(q, k, v, scale, causal, Oref, Lref, fp8=None):
    """scales_head over a whole (B, H, N, D) problem (``fp8``: (q codes,
    k codes, dq, dk) of the whole tensors)."""
    B, Hq, Nq, _ = q.shape
    G = Hq // k.shape[1]
    rows = np.arange(Nq)
    parts = {}
    for b in range(B):
        for h in range(Hq):
            f8 = None if fp8 is None else (fp8[0][b, h], fp8[1][b, h // G], fp8[2], fp8[3])
            r = scales_head(q[b, h], k[b, h // G], v[b, h // G], scale, causal, rows, Oref[b, h], Lref[b, h], f8)
            for key, val in r.items():
                parts.setdefault(key, np.empty((B, Hq) + val.shape))[b, h] = val
    return parts


def bar_violations(O, L, Oref, Lref, dtype, sc=None, scale_aware=True):
    """List of violated bars (empty when O, L pass) for one set of rows.
    ``sc``: scales(_head) of the same rows (the scale-aware output bar is
    skipped without it, and for fp32)."""
    sc = sc or {}
    bad = []
    if not np.isfinite(O).all():
        return ["non-finite or unwritten output"]
    err = float(np.abs(O - Oref).max()) if O.size else 0.0
    if err > TOL_O[dtype]:
        bad.append(f"max |dO| = {err:.3e} > {TOL_O[dtype]}")
    fin = np.isfinite(Lref)
    if not np.array_equal(np.isneginf(L), ~fin):
        bad.append("LSE -inf pattern differs")
    elif fin.any():
        d = np.abs(L[fin] - Lref[fin])
        lrel = float((d / np.maximum(1.0, np.abs(Lref[fin]))).max())
        if lrel > TOL_LSE_REL:
            bad.append(f"LSE rel err {lrel:.3e} > {TOL_LSE_REL}")
        lim_l = ABS_LSE + (sc["lse_extra"][fin] if "lse_extra" in sc else 0.0)
        if scale_aware and (d > lim_l).any():
            i = int(np.argmax(d - lim_l))
            bad.append(f"|dLSE| = {float(d[i]):.3e} > {float(np.broadcast_to(lim_l, d.shape)[i]):.3e} "
                       f"(scale-aware bar)")
    if scale_aware and "sigma" in sc and dtype != "f32" and O.size:
        lim = U_BF16 * np.abs(Oref) + SIGMAS * sc["sigma"] + sc.get("o_extra", 0.0) + 1e-7
        over = np.abs(O - Oref) > lim
        if over.any():
            i = np.unravel_index(int(np.argmax(np.abs(O - Oref) - lim)), O.shape)
            bad.append(f"{int(over.sum())} elements with |dO| > 2^-8 |O| + {SIGMAS:g} sigma, worst "
                       f"{abs(O[i] - Oref[i]):.3e} against {lim[i]:.3e} (scale-aware bar)")
    return bad


def round_bf16(x):
    """Round float64 values to the nearest bfloat16 (ties to even), as float64."""
    f = np.asarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).astype(np.float64)
