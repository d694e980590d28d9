"""attn_fwd_splitkv_noalloc (through the C ABI): the allocation-free variant
of attn_fwd_splitkv, whose partial results live in the library's fixed
per-GPU scratch area, against attn_fwd_splitkv with a caller workspace
(same kernels, same key ranges: bitwise equal) and against the fp64 oracle
(the stated and scale-aware bars).

Two calls in a row, the second on a smaller problem, so the second runs on
a scratch area that still holds the first call's partial results.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from bars import bar_violations
from exact_io_aware_attn_amd import attn as A
from exact_io_aware_attn_amd.inputs import Workload, make_inputs

pytestmark = pytest.mark.gpu


def note(msg):
    print(f"[gpu-case] {msg}", file=sys.stderr, flush=True)


CALLS = [
    # (B, Hq, Hkv, Nq, Nkv, D, causal, dtype, n_splits): the second is smaller
    (1, 32, 8, 256, 8192, 128, True, "bf16", 8),
    (1, 4, 2, 100, 1000, 64, False, "bf16", 3),
]


def _one(case, seed):
    B, Hq, Hkv, Nq, Nkv, D, causal, dt, ns = case
    note(f"attn_fwd_splitkv_noalloc {case}")
    w = Workload("noalloc", B, Hq, Hkv, Nq, Nkv, D, causal, dt, seed=seed)
    assert A.splitkv_workspace_bytes(B, Hq, Nq, D, ns) <= A.NOALLOC_SCRATCH_BYTES
    inp = make_inputs(w)
    q, k, v = (t.cuda() for t in inp)
    out = torch.full((B, Hq, Nq, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((B, Hq, Nq), float("nan"), dtype=torch.float32, device="cuda")
    A.fwd_splitkv_noalloc(q, k, v, ns, causal=causal, scale=w.scale, out=out, lse=lse)
    ref_o, ref_l = A.fwd_splitkv(q, k, v, ns, causal=causal, scale=w.scale)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref_o.view(torch.int16)), "O differs from attn_fwd_splitkv"
    assert torch.equal(lse.view(torch.int32), ref_l.view(torch.int32)), "LSE differs from attn_fwd_splitkv"
    O, L = out.float().cpu().double().numpy(), lse.cpu().double().numpy()
    G = Hq // Hkv
    qq, kk, vv = (t.to(torch.float64).numpy() for t in inp)
    rows = np.unique(np.concatenate([[0, Nq - 1], np.random.default_rng(seed).integers(0, Nq, 32)]))
    for b in range(B):
        for h in range(Hq):
            Oref, Lref = oracle.attention_head(qq[b, h], kk[b, h // G], vv[b, h // G], w.scale, causal, rows=rows)
            bad = bar_violations(O[b, h][rows], L[b, h][rows], Oref, Lref, dt)
            assert not bad, f"head {h}: " + "; ".join(bad)


def test_noalloc_two_calls_second_smaller():
    _one(CALLS[0], seed=31)
    _one(CALLS[1], seed=32)
