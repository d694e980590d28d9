"""GPU parity at the largest sizes the boundary accepts (include/attn.h: each
(batch, head) slab of q, k, v and o below 2^31 bytes, the range of the
kernels' 32-bit buffer offsets): slabs of 2^31 - 2 D bytes, so the last row
ends just below the limit and every tile grid has a ragged tail there, and
several heads, so whole tensors pass 2^31 bytes (64-bit slab bases).

Random inputs would hide an addressing fault at this size: a kernel reading
the wrong keys of a million random ones changes O and LSE by less than the
bars.  The inputs are therefore structured, in the manner of the oracle pin
"one-hot dominant logits select a V row": K and V are zero except at marker
keys spread over the slab (its first rows, its middle, its last rows), marker
m carries a one-hot key on channel m and a random value row, and each query
selects one marker through a score of 30 (natural units) on that channel,
so its output is that marker's value row to within about 1e-6, and every
other key has score 0.  A query that reads a wrong or wrapped row gets
another row (zeros or another marker).  The oracle is the plain float64
definition on the sampled rows (every key of them materialised); the bars
are the stated ones (2e-2 max-abs, LSE 1e-3 x max(1, |LSE|)).

Inputs are built on the device with torch operations (zeros, a seeded
normal draw for the value rows, index writes) and copied to the host for the
oracle; nothing comes from this library's kernels.
"""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
from bars import bar_violations
from exact_io_aware_attn_amd import attn as A

pytestmark = pytest.mark.gpu

SCORE = 30.0   # dominant score (natural units) of a query's chosen marker


def note(msg):
    print(f"[gpu-case] {msg}", file=sys.stderr, flush=True)


def max_rows(D, elt=2):
    """Largest row count whose slab of elt-byte elements stays below 2^31
    bytes."""
    return (1 << 31) // (elt * D) - 1


def marker_keys(Nkv, n):
    """n distinct marker positions spread over [0, Nkv): the first rows, the
    2^k boundaries and the last rows of the slab."""
    cand = [0, 1, 31, 32, 4095, 4096, (Nkv // 2) | 1, 1 << 20, (1 << 22) + 3, Nkv - 200, Nkv - 129, Nkv - 128,
            Nkv - 65, Nkv - 64, Nkv - 33, Nkv - 32, Nkv - 3, Nkv - 2, Nkv - 1]
    keys = sorted({j for j in cand if 0 <= j < Nkv})
    if len(keys) > n:
        keys = keys[:n // 2] + keys[len(keys) - (n - n // 2):]
    return np.asarray(keys, dtype=np.int64)


def check(O, L, Oref, Lref, label, dt="bf16"):
    bad = bar_violations(O, L, Oref, Lref, dt, scale_aware=False)
    note(f"  {label}: max |dO| = {np.abs(O - Oref).max():.3e}")
    assert not bad, f"{label}: " + "; ".join(bad)


@pytest.mark.parametrize("D,Hq,Hkv,Nq,causal,dt", [(128, 2, 1, 100, True, "bf16"), (320, 1, 1, 70, False, "bf16"),
                                                    (512, 2, 1, 40, True, "bf16"), (768, 2, 1, 70, False, "bf16"),
                                                    (1024, 1, 1, 70, False, "bf16"), (96, 2, 2, 50, True, "bf16"),
                                                    (128, 1, 1, 70, False, "f32")],
                         ids=["d128_gqa_causal", "d320", "d512_gqa_causal", "d768_gqa", "d1024", "d96_tiled",
                              "f32_d128_tiled"])
def test_longest_key_slab(D, Hq, Hkv, Nq, causal, dt):
    """K and V slabs just below 2^31 bytes (8 388 607 bf16 keys at D = 128
    down to 1 048 575 at D = 1024): the bf16 kernel (a small grid, 64-key
    tiles), the wide-head kernel (64-key tiles at D = 320, 32 at 512), the
    four-wave and the eight-wave split-D kernels, and the generic tiled
    kernel (bf16 D = 96, fp32) stream every key tile up to the limit."""
    elt = 4 if dt == "f32" else 2
    tdt = torch.float32 if dt == "f32" else torch.bfloat16
    Nkv = max_rows(D, elt)
    note(f"longest key slab: B=1 Hq={Hq} Hkv={Hkv} Nq={Nq} Nkv={Nkv} D={D} causal={causal} {dt}")
    dev = torch.device("cuda:0")
    scale = 1.0 / math.sqrt(D)
    marks = marker_keys(Nkv, min(D, 16))
    M = len(marks)
    g = torch.Generator(device=dev).manual_seed(D)
    k = torch.zeros(1, Hkv, Nkv, D, dtype=tdt, device=dev)
    v = torch.zeros(1, Hkv, Nkv, D, dtype=tdt, device=dev)
    mk = torch.from_numpy(marks).to(dev)
    for h in range(Hkv):
        k[0, h, mk, torch.arange(M, device=dev)] = 1.0
        v[0, h, mk] = torch.randn(M, D, generator=g, device=dev).to(tdt)
    # query i of head h picks a marker it can see: the last one visible
    # (head 0) or another visible one (head 1)
    q = torch.zeros(1, Hq, Nq, D, dtype=tdt, device=dev)
    off = Nkv - Nq
    for h in range(Hq):
        for i in range(Nq):
            vis = np.nonzero(marks <= (i + off if causal else Nkv - 1))[0]
            m = int(vis[-1]) if h == 0 else int(vis[(7 * i + 3) % len(vis)])
            q[0, h, i, m] = SCORE / scale
    o, lse = A.fwd(q, k, v, causal=causal, scale=scale)
    torch.cuda.synchronize()
    rows = np.unique(np.array([0, 1, Nq // 2, Nq - 2, Nq - 1]))
    kh = [k[0, h].double().cpu().numpy() for h in range(Hkv)]
    vh = [v[0, h].double().cpu().numpy() for h in range(Hkv)]
    G = Hq // Hkv
    for h in range(Hq):
        Oref, Lref = oracle.attention_head(q[0, h].double().cpu().numpy(), kh[h // G], vh[h // G], scale, causal,
                                           rows=rows)
        O = o[0, h, torch.from_numpy(rows).to(dev)].double().cpu().numpy()
        L = lse[0, h, torch.from_numpy(rows).to(dev)].double().cpu().numpy()
        check(O, L, Oref, Lref, f"head {h}", dt)


def test_longest_query_slab():
    """Q and O slabs of 2^31 - 256 bytes (8 388 607 rows at D = 128) in two
    heads (4 GiB tensors): 131 072 work-groups of the bf16 kernel (32-key
    tiles, three per CU), the last one ragged, write every row up to the
    limit; row i selects key (7 i + h) mod Nkv, one-hot keys on channel j."""
    D, Hq, Nkv = 128, 2, 77
    Nq = max_rows(D)
    note(f"longest query slab: B=1 Hq={Hq} Hkv={Hq} Nq={Nq} Nkv={Nkv} D={D}")
    dev = torch.device("cuda:0")
    scale = 1.0 / math.sqrt(D)
    g = torch.Generator(device=dev).manual_seed(7)
    k = torch.zeros(1, Hq, Nkv, D, dtype=torch.bfloat16, device=dev)
    k[0, :, torch.arange(Nkv, device=dev), torch.arange(Nkv, device=dev)] = 1.0
    v = torch.randn(1, Hq, Nkv, D, generator=g, device=dev).to(torch.bfloat16)
    q = torch.zeros(1, Hq, Nq, D, dtype=torch.bfloat16, device=dev)
    i = torch.arange(Nq, device=dev)
    for h in range(Hq):
        q[0, h, i, (7 * i + h) % Nkv] = SCORE / scale
    o, lse = A.fwd(q, k, v, causal=False, scale=scale)
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    rows = np.unique(np.concatenate([[0, 1, 127, 128, 1 << 22, Nq - 129, Nq - 128, Nq - 33, Nq - 32, Nq - 2, Nq - 1],
                                     rng.integers(0, Nq, 16)]))
    rt = torch.from_numpy(rows).to(dev)
    for h in range(Hq):
        Oref, Lref = oracle.attention_head(q[0, h, rt].double().cpu().numpy(), k[0, h].double().cpu().numpy(),
                                           v[0, h].double().cpu().numpy(), scale, False)
        check(o[0, h, rt].double().cpu().numpy(), lse[0, h, rt].double().cpu().numpy(), Oref, Lref, f"head {h}")


def test_longest_key_slab_e4m3():
    """e4m3 K and V slabs of 2^31 - 128 bytes (16 777 215 keys at D = 128,
    one byte per element): the direct-to-LDS kernel's K tiles and its
    register-staged V rows up to the limit.  Codes: one-hot keys 1.0, value
    rows of N(0, 1) draws rounded to e4m3, query code 352 on the marker's
    channel (score 31 with unit descales)."""
    D, Hq, Hkv, Nq = 128, 2, 1, 90
    Nkv = max_rows(D, 1)
    note(f"longest e4m3 key slab: B=1 Hq={Hq} Hkv={Hkv} Nq={Nq} Nkv={Nkv} D={D} causal=True")
    dev = torch.device("cuda:0")
    scale = 1.0 / math.sqrt(D)
    marks = marker_keys(Nkv, 16)
    M = len(marks)
    g = torch.Generator(device=dev).manual_seed(3)
    k = torch.zeros(1, Hkv, Nkv, D, dtype=torch.uint8, device=dev)
    v = torch.zeros(1, Hkv, Nkv, D, dtype=torch.uint8, device=dev)
    mk = torch.from_numpy(marks).to(dev)
    k[0, 0, mk, torch.arange(M, device=dev)] = 0x38                     # e4m3 1.0
    v[0, 0, mk] = torch.randn(M, D, generator=g, device=dev).to(torch.float8_e4m3fn).view(torch.uint8)
    q = torch.zeros(1, Hq, Nq, D, dtype=torch.uint8, device=dev)
    off = Nkv - Nq
    for h in range(Hq):
        for i in range(Nq):
            vis = np.nonzero(marks <= i + off)[0]
            m = int(vis[-1]) if h == 0 else int(vis[(5 * i + 1) % len(vis)])
            q[0, h, i, m] = 0x7B                                          # e4m3 352
    one = torch.ones(1, dtype=torch.float32, device=dev)
    q8, k8, v8 = (t.view(torch.float8_e4m3fn) for t in (q, k, v))
    o, lse = A.fwd_fp8(q8, k8, v8, one, one, one, causal=True, scale=scale)
    torch.cuda.synchronize()
    rows = np.array([0, 1, Nq // 2, Nq - 2, Nq - 1])
    rt = torch.from_numpy(rows).to(dev)
    # the oracle's decoding of every code, applied by table lookup (two
    # billion codes per tensor)
    table = oracle.e4m3fn_decode(np.arange(256, dtype=np.uint8))
    kh = table[k[0, 0].cpu().numpy()]
    vh = table[v[0, 0].cpu().numpy()]
    for h in range(Hq):
        Oref, Lref = oracle.attention_head(table[q[0, h].cpu().numpy()], kh, vh, scale, True, rows=rows)
        check(o[0, h, rt].double().cpu().numpy(), lse[0, h, rt].double().cpu().numpy(), Oref, Lref, f"head {h}")
