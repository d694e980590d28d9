"""GPU parity of the fp8 input pipeline (attn_quantize_fp8 and
attn_fwd_fp8_blocks, through the C ABI) against the fp64 oracle's
``quantize_blocks`` / ``dequantize_blocks`` / ``attention``, and its accuracy
against fp64 attention on the original bf16 inputs.

FA blog, section "FA3 — el momento Hopper": block quantisation (a scale per
64 x d tile) and a random orthogonal Hadamard-based rotation before
quantising, documented there to cut the fp8 error well below per-tensor fp8.
ZYFA article, section "The ZYFA accuracy work is the sleeper contribution":
rotating Q and K before quantisation roughly halves the input error.

Bars:
  * quantiser without rotation: codes and descales bit-exact (both sides take
    the float32 decisions: amax, 448 / amax, x * inv, nearest-even e4m3);
  * quantiser with rotation: the device's fast Walsh-Hadamard transform sums
    in float32, the oracle rotates in float64; every descale and code must lie
    in the range the float32 rotation's error bound admits
    (``fp8_bounds.rotated_code_intervals``), so a code may differ from the
    oracle's only where the oracle's value sits within that bound of an e4m3
    rounding boundary;
  * block-scaled attention on given codes and block descales: the fp8
    tolerance, 8e-2 max-abs on outputs of unit scale (these inputs have no
    outlier channels, |O| < 7), LSE 1e-3 * max(1, |LSE|);
  * the whole pipeline on the outlier recipe: outputs reach |O| ~ 30 (a
    sharp softmax picks out rows of V with outlier channels), where the bf16
    rounding of P and of O is relative, so 8e-2 * max(1, |O_ref|);
  * accuracy gate: against fp64 attention on the bf16 inputs, block scales
    lower the output RMS error to at most 0.75x that of per-tensor fp8, and
    rotating Q and K lowers it further to at most 0.7x of block scales alone
    (the oracle gives 0.32-0.53x and 0.39-0.50x over seeds 0-3).
"""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
from fp8_bounds import ordinal, rotated_code_intervals
from growing import growing_e4m3
from exact_io_aware_attn_amd import attn as A
from exact_io_aware_attn_amd.inputs import WORKLOADS, Workload, block_descales, make_inputs, quantize_e4m3

pytestmark = pytest.mark.gpu

TOL_FP8 = 8e-2
TOL_LSE = 1e-3


def note(msg):
    print(f"[gpu-case] {msg}", file=sys.stderr, flush=True)


def check_lse(L, Lref):
    fin = np.isfinite(Lref)
    assert np.array_equal(np.isneginf(L), ~fin), "LSE -inf pattern differs"
    if fin.any():
        lerr = (np.abs(L[fin] - Lref[fin]) / np.maximum(1.0, np.abs(Lref[fin]))).max()
        assert lerr <= TOL_LSE, f"LSE rel err {lerr:.3e}"


def bf16_recipe(B, Hq, Hkv, Nq, Nkv, D, causal=False, seed=0, frac=0.01):
    w = Workload("fp8blk", B, Hq, Hkv, Nq, Nkv, D, causal, "fp8blk", outlier_frac=frac, seed=seed)
    return w, make_inputs(w)


# ---- quantiser ----------------------------------------------------------------------

QUANT = [
    # (B, H, N, D)
    (1, 2, 200, 64),      # ragged last block
    (2, 3, 130, 128),     # zero block in the middle (rows 64..127)
    (1, 2, 100, 256),
    (1, 1, 1, 128),       # one row
    (1, 2, 64, 64),       # exactly one block
    (1, 4, 777, 128),
]


def quant_input(B, H, N, D, seed):
    _, (q, _, _, signs) = bf16_recipe(B, H, H, N, N, D, seed=seed)
    x = q.clone()
    if N >= 128:
        x[:, :, 64:128] = 0.0
        x[0, 0, 64, 0] = torch.tensor(-0.0, dtype=torch.bfloat16)
    return x, signs


@pytest.mark.parametrize("case", QUANT, ids=lambda c: "x".join(map(str, c)))
def test_quantize_plain_bit_exact(case):
    B, H, N, D = case
    note(f"quantize plain {case}")
    x, _ = quant_input(B, H, N, D, seed=3)
    codes, desc = A.quantize_fp8(x.cuda())
    torch.cuda.synchronize()
    c_ref, d_ref = oracle.quantize_blocks(x.to(torch.float64).numpy())
    d = desc.cpu().numpy()
    assert d.dtype == np.float32 and d.shape == d_ref.shape
    assert np.array_equal(d.view(np.uint32), d_ref.view(np.uint32)), "descales differ"
    c = codes.view(torch.uint8).cpu().numpy()
    bad = np.argwhere(c != c_ref)
    assert bad.size == 0, f"{len(bad)} codes differ, first at {bad[0]}: {c[tuple(bad[0])]:#x} vs {c_ref[tuple(bad[0])]:#x}"
    if N >= 128:
        assert (d[:, :, 1] == 1.0).all() and not (c[:, :, 64:128] & 0x7F).any()


@pytest.mark.parametrize("case", QUANT, ids=lambda c: "x".join(map(str, c)))
def test_quantize_rotated(case):
    """Rotated codes and descales within what the device's float32 rotation
    admits, element by element (``fp8_bounds.rotated_code_intervals``: a
    code may differ from the oracle's only where the oracle's value lies
    within the float32 rotation's error bound of an e4m3 rounding
    boundary)."""
    B, H, N, D = case
    note(f"quantize rotated {case}")
    x, signs = quant_input(B, H, N, D, seed=4)
    codes, desc = A.quantize_fp8(x.cuda(), signs.cuda())
    torch.cuda.synchronize()
    lo, hi, dlo, dhi = rotated_code_intervals(x.to(torch.float64).numpy(), signs.numpy().astype(np.float64))
    d = desc.cpu().numpy().astype(np.float64)
    assert ((dlo <= d) & (d <= dhi)).all(), "descale outside the float32 rotation's bound"
    c = ordinal(codes.view(torch.uint8).cpu().numpy())
    out = (c < lo) | (c > hi)
    assert not out.any(), f"{int(out.sum())} codes outside the admissible range, first at {np.argwhere(out)[0]}"
    c_ref, _ = oracle.quantize_blocks(x.to(torch.float64).numpy(), signs.numpy())
    note(f"  {int((c != ordinal(c_ref)).sum())} codes differ from the oracle's, {int((lo != hi).sum())} open of {c.size}")
    if N >= 128:
        assert (desc.cpu().numpy()[:, :, 1] == 1.0).all() and not (codes.view(torch.uint8).cpu().numpy()[:, :, 64:128] & 0x7F).any()


def test_quantize_rotation_is_orthogonal_on_device():
    """Decoded rotated codes times R^T give back x to e4m3 precision: the
    device applied R = diag(signs) H / sqrt(D), not another +-1 matrix."""
    x, signs = quant_input(1, 2, 256, 128, seed=5)
    codes, desc = A.quantize_fp8(x.cuda(), signs.cuda())
    torch.cuda.synchronize()
    y = oracle.dequantize_blocks(codes.view(torch.uint8).cpu().numpy(), desc.cpu().numpy())
    back = y @ oracle.rotation(signs.numpy()).T
    x64 = x.to(torch.float64).numpy()
    rel = np.sqrt(((back - x64) ** 2).sum() / (x64 ** 2).sum())
    assert rel < 0.04, f"relative reconstruction error {rel:.3e}"


# ---- block-scaled attention on given codes ---------------------------------------------

BLOCKS = [
    # (B, Hq, Hkv, Nq, Nkv, D, causal)
    (1, 2, 2, 200, 300, 128, True),
    (2, 4, 2, 130, 257, 64, False),
    (1, 2, 1, 100, 190, 256, True),
    (1, 2, 2, 64, 64, 128, False),
    (1, 2, 2, 1, 70, 128, True),
    (1, 3, 1, 333, 129, 64, True),
    (1, 2, 2, 257, 1000, 128, False),
    (1, 128, 32, 300, 400, 128, False),     # eight-wave work-groups
]


@pytest.mark.parametrize("case", BLOCKS, ids=lambda c: "x".join(map(str, c)))
def test_blocks_attention_parity(case):
    B, Hq, Hkv, Nq, Nkv, D, causal = case
    note(f"fwd_fp8_blocks {case}")
    w = Workload("fp8b", B, Hq, Hkv, Nq, Nkv, D, causal, "fp8", seed=9)
    q8, k8, v8, _ = make_inputs(w)
    ds = block_descales(w)
    exact = [oracle.dequantize_blocks(t.view(torch.uint8).numpy(), d) for t, d in zip((q8, k8, v8), ds)]
    dev = [t.cuda() for t in (q8, k8, v8)]
    ddev = [torch.from_numpy(d).cuda() for d in ds]
    O, L = A.fwd_fp8_blocks(*dev, *ddev, causal=causal, scale=w.scale)
    torch.cuda.synchronize()
    Oref, Lref = oracle.attention(*exact, scale=w.scale, causal=causal)
    O = O.float().cpu().numpy()
    assert np.isfinite(O).all()
    err = np.abs(O - Oref).max()
    assert err <= TOL_FP8, f"max |dO| = {err:.3e}"
    check_lse(L.cpu().numpy(), Lref)


@pytest.mark.parametrize("case", [(1, 2, 2, 150, 150, 128, True, 0.25), (1, 2, 1, 200, 300, 128, False, 0.1),
                                  (1, 2, 2, 200, 300, 64, True, 0.25), (1, 2, 2, 100, 190, 256, True, 0.1)],
                         ids=lambda c: "x".join(map(str, c)))
def test_blocks_growing_scores(case):
    """Block descales on scores that rise along the key axis: the rescale
    decision bounds the tile sum of the probabilities without the V block
    factor folded into them, and the K block factor changes the exponent's
    multiplier from one 64-key tile to the next."""
    B, Hq, Hkv, Nq, Nkv, D, causal, gain = case
    note(f"fwd_fp8_blocks growing {case}")
    q8, k8, v8, base = growing_e4m3(B, Hq, Hkv, Nq, Nkv, D, gain, seed=Nkv + D)
    rng = np.random.default_rng(Nq)
    ds = [(rng.uniform(0.5, 2.0, size=(B, H, (N + 63) // 64)) * d).astype(np.float32)
          for d, H, N in zip(base, (Hq, Hkv, Hkv), (Nq, Nkv, Nkv))]
    exact = [oracle.dequantize_blocks(t.view(torch.uint8).numpy(), d) for t, d in zip((q8, k8, v8), ds)]
    scale = 1.0 / math.sqrt(D)
    O, L = A.fwd_fp8_blocks(*(t.cuda() for t in (q8, k8, v8)), *(torch.from_numpy(d).cuda() for d in ds),
                            causal=causal, scale=scale)
    torch.cuda.synchronize()
    Oref, Lref = oracle.attention(*exact, scale=scale, causal=causal)
    O = O.float().cpu().numpy()
    assert np.isfinite(O).all()
    err = np.abs(O - Oref).max()
    assert err <= TOL_FP8, f"max |dO| = {err:.3e}"
    check_lse(L.cpu().numpy(), Lref)


def test_blocks_equal_descales_match_per_tensor_path():
    """All block descales equal to the per-tensor descale: the same result as
    attn_fwd_fp8 up to float32 rounding order."""
    w = Workload("fp8e", 1, 2, 2, 300, 300, 128, True, "fp8", seed=2, outlier_frac=0.01)
    q8, k8, v8, desc = make_inputs(w)
    dev = [t.cuda() for t in (q8, k8, v8)]
    nb = (300 + 63) // 64
    ddev = [torch.full((1, 2, nb), float(d), dtype=torch.float32, device="cuda:0") for d in desc]
    Ob, Lb = A.fwd_fp8_blocks(*dev, *ddev, causal=True, scale=w.scale)
    one = [torch.tensor([float(d)], dtype=torch.float32, device="cuda:0") for d in desc]
    Ot, Lt = A.fwd_fp8(*dev, *one, causal=True, scale=w.scale)
    torch.cuda.synchronize()
    Ob, Ot = Ob.float().cpu().numpy(), Ot.float().cpu().numpy()
    assert np.abs(Ob - Ot).max() <= 2e-2 * max(1.0, np.abs(Ot).max())
    assert np.abs(Lb.cpu().numpy() - Lt.cpu().numpy()).max() <= 1e-4 * max(1.0, np.abs(Lt.cpu().numpy()).max())


# ---- the whole pipeline -------------------------------------------------------------------

def device_pipeline(q, k, v, signs, causal, scale, rotate=True):
    sg = signs.cuda() if rotate else None
    cq, dq = A.quantize_fp8(q.cuda(), sg)
    ck, dk = A.quantize_fp8(k.cuda(), sg)
    cv, dv = A.quantize_fp8(v.cuda(), None)
    return A.fwd_fp8_blocks(cq, ck, cv, dq, dk, dv, causal=causal, scale=scale)


def oracle_pipeline_inputs(q, k, v, signs, rotate=True):
    s = signs.numpy() if rotate else None
    out = []
    for t, sg in zip((q, k, v), (s, s, None)):
        c, d = oracle.quantize_blocks(t.to(torch.float64).numpy(), sg)
        out.append(oracle.dequantize_blocks(c, d))
    return out


PIPE = [
    (1, 2, 2, 256, 256, 128, False),
    (1, 4, 1, 200, 300, 64, True),
    (1, 2, 2, 130, 190, 256, False),
    (2, 4, 2, 129, 700, 128, True),
]


@pytest.mark.parametrize("case", PIPE, ids=lambda c: "x".join(map(str, c)))
def test_pipeline_parity(case):
    B, Hq, Hkv, Nq, Nkv, D, causal = case
    note(f"fp8 pipeline {case}")
    w, (q, k, v, signs) = bf16_recipe(B, Hq, Hkv, Nq, Nkv, D, causal, seed=6)
    O, L = device_pipeline(q, k, v, signs, causal, w.scale)
    torch.cuda.synchronize()
    Oref, Lref = oracle.attention(*oracle_pipeline_inputs(q, k, v, signs), scale=w.scale, causal=causal)
    O = O.float().cpu().numpy()
    assert np.isfinite(O).all()
    excess = (np.abs(O - Oref) / np.maximum(1.0, np.abs(Oref))).max()
    assert excess <= TOL_FP8, f"max |dO| / max(1, |O|) = {excess:.3e}"
    check_lse(L.cpu().numpy(), Lref)


def test_accuracy_gate():
    """Block scales, then the rotation, each lower the error against fp64
    attention on the original bf16 inputs (shared Q/K outlier channels)."""
    w, (q, k, v, signs) = bf16_recipe(1, 4, 4, 512, 512, 128, seed=0)
    ref, _ = oracle.attention(*(t.to(torch.float64).numpy() for t in (q, k, v)), scale=w.scale)
    rmse = lambda o: float(np.sqrt(((o.float().cpu().numpy() - ref) ** 2).mean()))
    per_tensor = []
    for t in (q, k, v):
        c, d = quantize_e4m3(t.to(torch.float64).numpy())
        per_tensor += [c.cuda(), torch.tensor([float(d)], dtype=torch.float32, device="cuda:0")]
    Ot, _ = A.fwd_fp8(per_tensor[0], per_tensor[2], per_tensor[4], per_tensor[1], per_tensor[3], per_tensor[5],
                      scale=w.scale)
    Ob, _ = device_pipeline(q, k, v, signs, False, w.scale, rotate=False)
    Or, _ = device_pipeline(q, k, v, signs, False, w.scale, rotate=True)
    torch.cuda.synchronize()
    et, eb, er = rmse(Ot), rmse(Ob), rmse(Or)
    note(f"output RMS error vs fp64: per-tensor {et:.4f}, block {eb:.4f}, block + rotation {er:.4f}")
    assert eb <= 0.75 * et, (et, eb)
    assert er <= 0.7 * eb, (eb, er)


def test_full_size_sampled():
    """The benchmarked problem (24 heads x 16K x 16K, D = 128): the device
    pipeline against the oracle pipeline on sampled rows."""
    w = WORKLOADS["fp8_blocks_outlier"]
    note(f"{w.name} full size")
    q, k, v, signs = make_inputs(w)
    O, L = device_pipeline(q, k, v, signs, w.causal, w.scale)
    torch.cuda.synchronize()
    O = O.float().cpu().numpy()
    L = L.cpu().numpy()
    assert np.isfinite(O).all() and np.isfinite(L).all()
    rng = np.random.default_rng(1)
    worst = 0.0
    G = w.Hq // w.Hkv
    for hq in [0, w.Hq - 1] + [int(h) for h in rng.integers(0, w.Hq, 2)]:
        # blocks never span heads: quantising one head's slab alone is exact
        hk = hq // G
        xq, xk, xv = oracle_pipeline_inputs(q[:, hq:hq + 1], k[:, hk:hk + 1], v[:, hk:hk + 1], signs)
        rows = np.unique(np.concatenate([[0, w.Nq - 1], rng.integers(0, w.Nq, 24)]))
        Oref, Lref = oracle.attention_head(xq[0, 0], xk[0, 0], xv[0, 0], w.scale, w.causal, rows=rows)
        ex = (np.abs(O[0, hq][rows] - Oref) / np.maximum(1.0, np.abs(Oref))).max()
        worst = max(worst, ex)
        check_lse(L[0, hq][rows], Lref)
    note(f"{w.name}: worst sampled max|dO| / max(1, |O|) = {worst:.3e}")
    assert worst <= TOL_FP8
