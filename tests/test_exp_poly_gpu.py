"""GPU parity of the polynomial-exponential variant (attn_fwd_exp_poly
through the C ABI): its probabilities differ from exp by at most 8.6e-5
relative (the cubic's bound, pinned in the oracle tests), below bf16
rounding, so it is held to the exact bf16 bar against the exact oracle
(2e-2 max-abs, LSE 1e-3 x max(1, |LSE|)), and to 2^-7 x max(1, |O|) against
the exp kernel's output (one bf16 step of O plus the polynomial's error).
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from exact_io_aware_attn_amd import attn as A
from exact_io_aware_attn_amd.inputs import WORKLOADS, Workload, make_inputs

pytestmark = pytest.mark.gpu


def note(msg):
    print(f"[gpu-case] {msg}", file=sys.stderr, flush=True)


CASES = [
    (1, 2, 2, 200, 300, 128, True),
    (2, 4, 2, 130, 257, 64, False),
    (1, 2, 1, 333, 129, 128, True),     # rows without keys
    (1, 2, 2, 1, 70, 128, True),
    (1, 2, 2, 257, 1000, 128, False),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "x".join(map(str, c)))
def test_exp_poly_parity(case):
    B, Hq, Hkv, Nq, Nkv, D, causal = case
    note(f"fwd_exp_poly {case}")
    w = Workload("poly", B, Hq, Hkv, Nq, Nkv, D, causal, "bf16", seed=2)
    q, k, v = make_inputs(w)
    dev = [t.cuda() for t in (q, k, v)]
    O, L = A.fwd_exp_poly(*dev, causal=causal, scale=w.scale)
    Oe, _ = A.fwd(*dev, causal=causal, scale=w.scale)
    torch.cuda.synchronize()
    O, L, Oe = O.float().cpu().numpy(), L.cpu().numpy(), Oe.float().cpu().numpy()
    Oref, Lref = oracle.attention(*(t.to(torch.float64).numpy() for t in (q, k, v)), w.scale, causal)
    assert np.isfinite(O).all()
    assert np.abs(O - Oref).max() <= 2e-2
    fin = np.isfinite(Lref)
    assert np.array_equal(np.isneginf(L), ~fin)
    if fin.any():
        assert (np.abs(L[fin] - Lref[fin]) / np.maximum(1.0, np.abs(Lref[fin]))).max() <= 1e-3
    d = (np.abs(O - Oe) / np.maximum(1.0, np.abs(Oe))).max()
    note(f"  max |O - O_exp| / max(1, |O|) = {d:.3e}")
    assert d <= 2.0 ** -7


@pytest.mark.parametrize("case", [(1, 2, 1, 150, 300, 128, False), (1, 2, 2, 200, 200, 128, True),
                                  (1, 2, 2, 130, 260, 64, True)], ids=lambda c: "x".join(map(str, c)))
def test_exp_poly_growing_scores(case):
    """Scores that grow by a quarter per key (channel 0: 4 in every query, a
    j in key j): the rescale path runs on (almost) every 64-key tile."""
    B, Hq, Hkv, Nq, Nkv, D, causal = case
    note(f"fwd_exp_poly growing {case}")
    w = Workload("polygrow", B, Hq, Hkv, Nq, Nkv, D, causal, "bf16", value_scale=0.5, seed=Nkv)
    q, k, v = make_inputs(w)
    q, k = q.float(), k.float()
    q[..., 0] = 4.0
    k[..., 0] = (D ** 0.5 / 16.0) * torch.arange(Nkv, dtype=torch.float32)
    q, k = q.to(torch.bfloat16), k.to(torch.bfloat16)
    O, L = A.fwd_exp_poly(*(t.cuda() for t in (q, k, v)), causal=causal, scale=w.scale)
    torch.cuda.synchronize()
    O, L = O.float().cpu().numpy(), L.cpu().numpy()
    Oref, Lref = oracle.attention(*(t.to(torch.float64).numpy() for t in (q, k, v)), w.scale, causal)
    assert np.isfinite(O).all()
    assert np.abs(O - Oref).max() <= 2e-2
    fin = np.isfinite(Lref)
    assert np.array_equal(np.isneginf(L), ~fin)
    assert (np.abs(L[fin] - Lref[fin]) / np.maximum(1.0, np.abs(Lref[fin]))).max() <= 1e-3


def test_exp_poly_full_size_sampled():
    w = WORKLOADS["prefill_causal_bf16"]
    note(f"{w.name} polynomial exp, full size")
    q, k, v = make_inputs(w)
    dev = [t.cuda() for t in (q, k, v)]
    O, L = A.fwd_exp_poly(*dev, causal=True, scale=w.scale)
    torch.cuda.synchronize()
    O, L = O.float().cpu().numpy(), L.cpu().numpy()
    rng = np.random.default_rng(5)
    worst = 0.0
    for b, h in [(0, 0), (w.B - 1, w.Hq - 1), (int(rng.integers(w.B)), int(rng.integers(w.Hq)))]:
        rows = np.unique(np.concatenate([[0, w.Nq - 1], rng.integers(0, w.Nq, 24)]))
        Oref, Lref = oracle.attention_head(q[b, h].double().numpy(), k[b, h].double().numpy(),
                                           v[b, h].double().numpy(), w.scale, True, rows=rows)
        worst = max(worst, float(np.abs(O[b, h][rows] - Oref).max()))
        assert (np.abs(L[b, h][rows] - Lref) / np.maximum(1.0, np.abs(Lref))).max() <= 1e-3
    note(f"  worst sampled max |dO| = {worst:.3e}")
    assert worst <= 2e-2
