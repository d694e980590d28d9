"""GPU parity of the key-range path: attn_fwd_partial, attn_merge and
attn_fwd_splitkv (through the C ABI) against the fp64 oracle's
``attention_range`` / ``merge`` / ``attention``.

Covers every kernel family (D = 64/128 direct-to-LDS, 192..512 wide-head,
576..1024 split-D, fp32 and other D on the tiled kernel, e4m3), ranges that
start and end inside a tile, ranges a causal row does not reach (O = 0,
LSE = -inf), splits that are empty, GQA and cross attention.

Tolerances as the main parity tests for the merged result (bf16 2e-2, fp8
8e-2, fp32 1e-4 max-abs, LSE 1e-3 * max(1, |LSE|)).  The partial outputs are
float32 normalised over the range: same bounds.  The merge alone runs in
float32 on float32 inputs: 1e-5 (float32 output) and bf16 rounding (bf16
output).
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from bars import bar_violations, scales, scales_head
from exact_io_aware_attn_amd import attn as A
from exact_io_aware_attn_amd.inputs import Workload, make_inputs

pytestmark = pytest.mark.gpu



def note(msg):
    print(f"[gpu-case] {msg}", file=sys.stderr, flush=True)


def gpu_and_oracle_inputs(w):
    """Device q, k, v (e4m3 codes for fp8), the descale tensors (None unless
    fp8) and the exact float64 values the kernels see."""
    inp = make_inputs(w)
    if w.dtype == "fp8":
        q8, k8, v8, desc = inp
        exact = tuple(oracle.e4m3fn_decode(t.view(torch.uint8).numpy()) * np.float64(d)
                      for t, d in zip((q8, k8, v8), desc))
        dev = tuple(t.cuda() for t in (q8, k8, v8))
        descales = tuple(torch.tensor([float(d)], dtype=torch.float32, device="cuda:0") for d in desc)
    else:
        exact = tuple(t.to(torch.float64).numpy() for t in inp)
        dev = tuple(t.cuda() for t in inp)
        descales = None
    return dev, descales, exact


def check(O, L, Oref, Lref, dtype, sc=None):
    """The stated and the scale-aware bars (``bars.py``; the output bar
    where the error scales ``sc`` are given)."""
    bad = bar_violations(O, L, Oref, Lref, dtype, sc=sc)
    assert not bad, "; ".join(bad)


PARTIAL = [
    # (B, Hq, Hkv, Nq, Nkv, D, causal, dtype, kv_begin, kv_end)
    (1, 2, 1, 200, 300, 128, True, "bf16", 70, 250),     # starts and ends inside tiles
    (1, 2, 2, 150, 150, 128, True, "bf16", 100, 150),    # early rows see none of the range
    (2, 4, 2, 90, 400, 64, False, "bf16", 0, 400),
    (1, 2, 2, 130, 330, 64, True, "bf16", 33, 34),       # one key
    (1, 2, 1, 140, 260, 256, True, "bf16", 64, 200),     # wide kernel, 64-key tiles
    (1, 2, 2, 100, 300, 512, False, "bf16", 17, 290),
    (1, 2, 2, 70, 200, 768, True, "bf16", 40, 200),      # split-D
    (1, 2, 1, 65, 130, 1024, False, "bf16", 31, 97),
    (1, 2, 1, 65, 130, 416, True, "bf16", 31, 97),       # split-D at the layout of D + 32
    (1, 2, 2, 90, 170, 96, True, "bf16", 50, 120),       # tiled kernel
    (1, 2, 2, 80, 150, 128, True, "f32", 20, 140),
    (1, 2, 2, 120, 260, 128, False, "fp8", 45, 201),
    (1, 2, 2, 100, 100, 128, True, "bf16", 0, 0),        # empty range
]


@pytest.mark.parametrize("case", PARTIAL, ids=lambda c: "B{}_Hq{}_Hkv{}_Nq{}_Nkv{}_D{}_{}_{}_[{},{})".format(
    *c[:6], "causal" if c[6] else "full", *c[7:]))
def test_partial_parity(case):
    B, Hq, Hkv, Nq, Nkv, D, causal, dt, kb, ke = case
    w = Workload("partial", B, Hq, Hkv, Nq, Nkv, D, causal, dt, seed=sum(case[:6]) + kb)
    note(f"partial {case}")
    (q, k, v), desc, (qe, ke_, ve) = gpu_and_oracle_inputs(w)
    o, lse = A.fwd_partial(q, k, v, kb, ke, causal=causal, scale=w.scale, descales=desc)
    torch.cuda.synchronize()
    Oref, Lref = oracle.attention_range(qe, ke_, ve, w.scale, causal, kb, ke)
    check(o.cpu().double().numpy(), lse.cpu().double().numpy(), Oref, Lref, dt)


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("P,D", [(1, 64), (3, 128), (7, 1024), (16, 32)])
def test_merge_parity(P, D, out_dtype):
    note(f"merge P={P} D={D} {out_dtype}")
    rng = np.random.default_rng(P * 1000 + D)
    B, Hq, Nq = 2, 3, 37
    Op = rng.standard_normal((P, B, Hq, Nq, D)).astype(np.float32)
    Lp = (rng.standard_normal((P, B, Hq, Nq)) * 4).astype(np.float32)
    # rows empty in some parts, and one row empty in every part
    Lp[rng.random((P, B, Hq, Nq)) < 0.2] = -np.inf
    Lp[:, 0, 0, 5] = -np.inf
    Op[np.isneginf(Lp)] = 0.0
    o, lse = A.merge(torch.from_numpy(Op).cuda(), torch.from_numpy(Lp).cuda(), out_dtype=out_dtype)
    torch.cuda.synchronize()
    Oref, Lref = oracle.merge(Op.astype(np.float64), Lp.astype(np.float64))
    tol = 1e-5 if out_dtype == torch.float32 else 2e-2
    O = o.float().cpu().double().numpy()
    assert np.isfinite(O).all()
    assert np.abs(O - Oref).max() <= tol
    L = lse.cpu().double().numpy()
    fin = np.isfinite(Lref)
    assert np.array_equal(np.isneginf(L), ~fin)
    assert (np.abs(L[fin] - Lref[fin]) / np.maximum(1.0, np.abs(Lref[fin]))).max() <= 1e-5
    assert np.all(O[0, 0, 5] == 0.0)


SPLITKV = [
    # (B, Hq, Hkv, Nq, Nkv, D, causal, dtype, n_splits)
    (1, 2, 1, 200, 1000, 128, True, "bf16", 4),
    (1, 4, 2, 64, 2000, 128, False, "bf16", 7),
    (1, 2, 2, 300, 300, 64, True, "bf16", 16),         # more splits than 64-key tiles per row
    (1, 2, 2, 50, 700, 256, False, "bf16", 3),
    (1, 2, 1, 129, 900, 512, True, "bf16", 5),
    (1, 2, 2, 64, 500, 1024, False, "bf16", 4),
    (1, 2, 2, 100, 640, 160, True, "bf16", 2),
    (1, 2, 2, 90, 333, 64, False, "f32", 3),
    (1, 2, 2, 100, 1200, 128, False, "fp8", 6),
    (1, 2, 2, 120, 100, 128, True, "bf16", 1),          # Nq > Nkv: keyless rows, one split
    (1, 32, 8, 300, 4000, 128, False, "bf16", 8),       # 512 eight-wave work-groups over the ranges
    (1, 32, 8, 300, 4000, 128, True, "bf16", 8),        # causal: eight waves over 4 GQA heads per range
    (1, 32, 8, 300, 4000, 128, False, "fp8", 8),
]


@pytest.mark.parametrize("case", SPLITKV, ids=lambda c: "B{}_Hq{}_Hkv{}_Nq{}_Nkv{}_D{}_{}_{}_s{}".format(
    *c[:6], "causal" if c[6] else "full", *c[7:]))
def test_splitkv_parity(case):
    B, Hq, Hkv, Nq, Nkv, D, causal, dt, ns = case
    w = Workload("splitkv", B, Hq, Hkv, Nq, Nkv, D, causal, dt, seed=sum(case[:6]) + ns)
    note(f"splitkv {case}")
    (q, k, v), desc, (qe, ke, ve) = gpu_and_oracle_inputs(w)
    o, lse = A.fwd_splitkv(q, k, v, ns, causal=causal, scale=w.scale, descales=desc)
    torch.cuda.synchronize()
    Oref, Lref = oracle.attention(qe, ke, ve, w.scale, causal)
    f8 = None
    if dt == "fp8":
        q8, k8, _, dsc = make_inputs(w)
        f8 = (oracle.e4m3fn_decode(q8.view(torch.uint8).numpy()), oracle.e4m3fn_decode(k8.view(torch.uint8).numpy()),
              dsc[0], dsc[1])
    check(o.float().cpu().double().numpy(), lse.cpu().double().numpy(), Oref, Lref, dt,
          scales(qe, ke, ve, w.scale, causal, Oref, Lref, f8))


def test_splitkv_matches_plain_call():
    """Same inputs through attn_fwd and attn_fwd_splitkv: both within the
    bf16 bound of each other, and the split path is bitwise repeatable."""
    w = Workload("splitkv_rep", 1, 4, 1, 256, 3000, 128, True, "bf16", seed=3)
    (q, k, v), _, _ = gpu_and_oracle_inputs(w)
    o1, l1 = A.fwd(q, k, v, causal=True)
    o2, l2 = A.fwd_splitkv(q, k, v, 8, causal=True)
    o3, l3 = A.fwd_splitkv(q, k, v, 8, causal=True)
    torch.cuda.synchronize()
    assert (o1.float() - o2.float()).abs().max().item() <= 2e-2
    assert (l1 - l2).abs().max().item() <= 1e-3 * max(1.0, l1.abs().max().item())
    assert torch.equal(o2.view(torch.int16), o3.view(torch.int16))
    assert torch.equal(l2.view(torch.int32), l3.view(torch.int32))


@pytest.mark.parametrize("name", ["chunk_prefill_splitkv_bf16", "chunk_prefill_bf16"])
def test_chunk_prefill_full_size_sampled(name):
    """The bench's chunked-prefill workloads at full size, in the launch
    configuration it times (split into extra["n_splits"] key ranges or not),
    against the oracle on sampled rows of a few heads."""
    from exact_io_aware_attn_amd.inputs import WORKLOADS
    w = WORKLOADS[name]
    note(f"{name} full size, sampled rows")
    (q, k, v), _, _ = gpu_and_oracle_inputs(w)
    ns = int(w.extra.get("n_splits", 0))
    if ns:
        o, lse = A.fwd_splitkv(q, k, v, ns, causal=w.causal, scale=w.scale)
    else:
        o, lse = A.fwd(q, k, v, causal=w.causal, scale=w.scale)
    torch.cuda.synchronize()
    O = o.float().cpu().double().numpy()
    L = lse.cpu().double().numpy()
    assert np.isfinite(O).all() and not np.isnan(L).any()
    qh, kh, vh = (t.cpu() for t in (q, k, v))
    rng = np.random.default_rng(5)
    G = w.Hq // w.Hkv
    for b, hq in [(0, 0), (w.B - 1, w.Hq - 1), (0, int(rng.integers(w.Hq)))]:
        rows = np.unique(np.concatenate([[0, w.Nq - 1], rng.integers(0, w.Nq, 40)]))
        args = (qh[b, hq].double().numpy(), kh[b, hq // G].double().numpy(), vh[b, hq // G].double().numpy())
        Oref, Lref = oracle.attention_head(*args, w.scale, w.causal, rows=rows)
        check(O[b, hq][rows], L[b, hq][rows], Oref, Lref, w.dtype,
              scales_head(*args, w.scale, w.causal, rows, Oref, Lref))
