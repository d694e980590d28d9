"""GPU parity of the backward pass (attn_bwd through the C ABI) against the
oracle's gradients (``oracle.attention_backward``, the chain rule through
the forward definition in float64).

Inputs: Q, K, V of the bf16 recipe and dO standard normal in bf16
(``inputs.make_grad``); O and LSE come from the library's own forward pass,
as a training step would pass them.

Tolerance (the pages state none for gradients; derived from the arithmetic):
the kernels round P and dS to bf16 (relative 2^-9) before the products, and
delta = dO . O uses the bf16 forward output; every product accumulates in
float32.  The bound is 2e-2 of each gradient's largest magnitude, about ten
bf16 roundings of the largest term, checked element by element over dQ, dK
and dV; rows that see no key must have dQ exactly 0.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from exact_io_aware_attn_amd import attn as A
from exact_io_aware_attn_amd.inputs import WORKLOADS, Workload, make_grad, make_inputs

pytestmark = pytest.mark.gpu

TOL = 2e-2


def note(msg):
    print(f"[gpu-case] {msg}", file=sys.stderr, flush=True)


def run_bwd(w):
    q, k, v = make_inputs(w)
    g = make_grad(w)
    dev = [t.cuda() for t in (q, k, v, g)]
    O, L = A.fwd(dev[0], dev[1], dev[2], causal=w.causal, scale=w.scale)
    dq, dk, dv = A.bwd(dev[0], dev[1], dev[2], O, L, dev[3], causal=w.causal, scale=w.scale)
    torch.cuda.synchronize()
    return (q, k, v, g), tuple(t.float().cpu().numpy() for t in (dq, dk, dv))


def rel_err(x, ref):
    return float(np.abs(x - ref).max()) / max(float(np.abs(ref).max()), 1e-30)


def zero_gradient_bound(q, k, v, g, scale, causal):
    """Absolute bounds on |dQ| and |dK| where the exact gradients are 0.

    When every visible row sees one key, P = 1 and delta = dO . O = dP, so dS
    = P (dP - delta) cancels to 0 exactly.  The kernels form dP (a matrix
    product) and delta (the prep launch) as float32 sums of the same D
    products in different orders; each differs from the exact value by at
    most D 2^-24 max|dP| (the standard bound for recursive summation), so
    |dS| <= 2 D 2^-24 max|dP| and dQ = scale dS K, dK = scale dS^T Q are
    bounded by that times scale max|K| Nkv and scale max|Q| Nq."""
    mask = oracle.visible_mask(q.shape[2], k.shape[2], causal)
    group = q.shape[1] // k.shape[1]
    vv = np.repeat(v.astype(np.float64), group, axis=1)
    dp = np.abs(np.einsum("bhid,bhjd->bhij", g.astype(np.float64), vv))[..., mask].max()
    eds = 2 * q.shape[3] * 2.0**-24 * dp
    return (abs(scale) * eds * np.abs(k).max() * k.shape[2], abs(scale) * eds * np.abs(q).max() * q.shape[2])


CASES = [
    # (B, Hq, Hkv, Nq, Nkv, D, causal)
    (1, 2, 2, 200, 300, 128, True),       # ragged, causal with Nq < Nkv
    (2, 4, 2, 130, 257, 64, False),       # GQA, ragged key tile
    (1, 2, 1, 333, 129, 128, True),       # Nq > Nkv: the first rows see no key
    (1, 2, 2, 1, 70, 128, True),          # one query row
    (1, 3, 1, 65, 65, 64, True),          # MQA
    (1, 2, 2, 257, 1000, 128, False),     # cross attention, several key work-groups
    (1, 2, 2, 64, 64, 128, False),        # exactly one tile
    (1, 4, 4, 513, 513, 128, True),       # several query and key tiles on the diagonal
    (1, 2, 2, 300, 1, 64, True),          # one key
    # D = 256 (its own dK/dV kernel)
    (1, 2, 2, 200, 300, 256, True),
    (2, 4, 2, 130, 257, 256, False),
    (1, 2, 1, 333, 129, 256, True),
    (1, 4, 4, 513, 513, 256, True),
    # D = 512 (each key or query block split between two waves)
    (1, 2, 2, 200, 300, 512, True),
    (2, 4, 2, 130, 257, 512, False),      # GQA, ragged, several key work-groups
    (1, 2, 1, 333, 129, 512, True),       # the first rows see no key
    (1, 2, 2, 1, 70, 512, True),          # one query row
    (1, 2, 2, 300, 1, 512, True),         # one key
    (1, 3, 1, 97, 97, 512, True),         # MQA, one query tile of each pair ragged
    (1, 2, 2, 256, 256, 512, True),       # whole tiles on the diagonal
    # the other multiples of 64 on the split kernels (rows of 24, 40, 48 and
    # 56 16-byte chunks; the prep kernel with idle lanes)
    (1, 2, 2, 200, 300, 192, True),
    (2, 4, 2, 130, 257, 320, False),
    (1, 2, 1, 333, 129, 384, True),
    (1, 3, 1, 97, 97, 448, True),
    (1, 2, 2, 1, 70, 384, True),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "x".join(map(str, c)))
def test_bwd_parity(case):
    B, Hq, Hkv, Nq, Nkv, D, causal = case
    note(f"bwd {case}")
    w = Workload("bwd", B, Hq, Hkv, Nq, Nkv, D, causal, "bf16", seed=3)
    (q, k, v, g), (dq, dk, dv) = run_bwd(w)
    ref = oracle.attention_backward(*(t.to(torch.float64).numpy() for t in (q, k, v, g)), scale=w.scale,
                                    causal=causal)
    zero_bound = None
    for name, x, r in zip(("dQ", "dK", "dV"), (dq, dk, dv), ref):
        assert np.isfinite(x).all(), f"{name}: non-finite values"
        if np.abs(r).max() == 0 and name != "dV":
            # an exact cancellation (one visible key per row): no relative
            # error to take, only the float32 rounding of dP - delta
            if zero_bound is None:
                zero_bound = dict(zip(("dQ", "dK"), zero_gradient_bound(
                    *(t.float().numpy() for t in (q, k, v, g)), w.scale, causal)))
            m = float(np.abs(x).max())
            note(f"  {name}: exact value 0, max |x| = {m:.3e} (bound {zero_bound[name]:.3e})")
            assert m <= zero_bound[name], f"{name}: {m:.3e} > {zero_bound[name]:.3e}"
            continue
        e = rel_err(x, r)
        note(f"  {name}: max |err| / max |ref| = {e:.3e}")
        assert e <= TOL, f"{name}: {e:.3e} > {TOL}"
    seen = oracle.visible_mask(Nq, Nkv, causal).any(axis=1)
    assert (dq[:, :, ~seen] == 0).all(), "rows without keys must get dQ = 0"


@pytest.mark.parametrize("D", [128, 256, 512])
def test_bwd_deterministic(D):
    w = Workload("bwd_det", 1, 4, 2, 300, 300, D, True, "bf16", seed=5)
    q, k, v = (t.cuda() for t in make_inputs(w))
    g = make_grad(w).cuda()
    O, L = A.fwd(q, k, v, causal=True, scale=w.scale)
    first = A.bwd(q, k, v, O, L, g, causal=True, scale=w.scale)
    second = A.bwd(q, k, v, O, L, g, causal=True, scale=w.scale)
    torch.cuda.synchronize()
    for a, b in zip(first, second):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("D", [64, 256, 512])
def test_bwd_scale_variants(D):
    """Scale 0 (uniform P: dQ = dK = 0) and a negative scale."""
    w = Workload("bwd_sc", 1, 2, 2, 150, 170, D, True, "bf16", seed=7)
    q, k, v = make_inputs(w)
    g = make_grad(w)
    dev = [t.cuda() for t in (q, k, v, g)]
    for sc in (0.0, -0.11):
        note(f"bwd D={D} scale={sc}")
        O, L = A.fwd(dev[0], dev[1], dev[2], causal=True, scale=sc)
        dq, dk, dv = A.bwd(dev[0], dev[1], dev[2], O, L, dev[3], causal=True, scale=sc)
        torch.cuda.synchronize()
        ref = oracle.attention_backward(*(t.to(torch.float64).numpy() for t in (q, k, v, g)), scale=sc, causal=True)
        for name, x, r in zip(("dQ", "dK", "dV"), (dq, dk, dv), ref):
            x = x.float().cpu().numpy()
            if np.abs(r).max() == 0:
                assert (x == 0).all(), name
            else:
                assert rel_err(x, r) <= TOL, (sc, name, rel_err(x, r))


# (Hq, Hkv, D); B = 1, N = 4096, causal
FULL_SIZE = {"causal_d256": (8, 8, 256), "gqa_causal_d512": (32, 8, 512)}


# bwd_causal_bf16_d512: 32 heads are enough work for the dK/dV launch to
# pair its causal key tiles
@pytest.mark.parametrize("name", ["prefill_causal_bf16", "causal_d256", "bwd_causal_bf16_d512", "gqa_causal_d512"])
def test_bwd_full_size_sampled(name):
    """The benchmarked problem (B4 H32 N4096 D128, causal), B1 H8 N4096 D256,
    B1 H32 N4096 D512 and its GQA form with 8 KV heads (causal): for three
    sampled KV heads, dQ of every query head of the group against the
    oracle's per-head gradients, and dK, dV against their sums over the
    group."""
    if name in WORKLOADS:
        w = WORKLOADS[name]
    else:
        Hq, Hkv, D = FULL_SIZE[name]
        w = Workload(name, 1, Hq, Hkv, 4096, 4096, D, True, "bf16")
    note(f"{w.name} backward, full size")
    (q, k, v, g), (dq, dk, dv) = run_bwd(w)
    rng = np.random.default_rng(2)
    G = w.Hq // w.Hkv
    # three KV heads; every query head of each one's group
    kv_heads = [(0, 0), (w.B - 1, w.Hkv - 1), (int(rng.integers(w.B)), int(rng.integers(w.Hkv)))]
    worst = 0.0
    for b, hk in kv_heads:
        kh, vh = (t[b, hk].to(torch.float64).numpy() for t in (k, v))
        sum_k = sum_v = 0.0
        for hq in range(hk * G, (hk + 1) * G):
            r_q, r_k, r_v = oracle.attention_backward_head(q[b, hq].to(torch.float64).numpy(), kh, vh,
                                                           g[b, hq].to(torch.float64).numpy(), scale=w.scale,
                                                           causal=w.causal)
            worst = max(worst, rel_err(dq[b, hq], r_q))
            sum_k = sum_k + r_k
            sum_v = sum_v + r_v
        worst = max(worst, rel_err(dk[b, hk], sum_k), rel_err(dv[b, hk], sum_v))
    note(f"{w.name}: worst max |err| / max |ref| over 3 KV heads = {worst:.3e}")
    assert worst <= TOL
