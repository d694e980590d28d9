"""Bitwise determinism of repeat launches, for every forward kernel
configuration (the ZYFA article, "The ZYFA accuracy work is the sleeper
contribution": outputs identical in every launch).

No kernel here uses atomics or a reduction whose order depends on timing,
so two launches on the same inputs must agree bit for bit, O and LSE.  Each
case runs the configuration the dispatcher picks for its shape: the bf16
kernel of head dims 64 and 128 with 64-key tiles (small grids) and with
32-key tiles at three waves per SIMD (grids of at least three work-groups
per compute unit), with and without causal tile pairing; the wide-head
kernel (64- and 32-key tiles); the four-wave split-D kernel (D = 768, and an
odd multiple of 32 on its padded layout) and the eight-wave one (D = 1024);
the generic tiled kernel; the e4m3 path with per-tensor and with block
descales; the e4m3-probability kernel, exact and Lean P codes.  The
backward's determinism is tested with its parity tests.
"""
import sys

import pytest
import torch

from exact_io_aware_attn_amd import attn as A
from exact_io_aware_attn_amd.inputs import Workload, block_descales, make_inputs

pytestmark = pytest.mark.gpu


def note(msg):
    print(f"[gpu-case] {msg}", file=sys.stderr, flush=True)


def same(a, b):
    if a.dtype == torch.bfloat16:
        return torch.equal(a.view(torch.int16), b.view(torch.int16))
    return torch.equal(a.view(torch.int32), b.view(torch.int32))


def twice(fn):
    o1, l1 = fn()
    o2, l2 = fn()
    torch.cuda.synchronize()
    assert torch.isfinite(o1.float()).all()
    assert same(o1, o2), "O differs between launches"
    assert same(l1, l2), "LSE differs between launches"


BF16 = [
    # (B, Hq, Hkv, Nq, Nkv, D, causal): kernel configuration
    (1, 8, 2, 700, 901, 128, True),      # direct-to-LDS, 64-key tiles (small grid)
    (1, 64, 64, 2048, 2048, 128, True),  # 32-key tiles, 1024 work-groups, unpaired
    (2, 64, 64, 4096, 4096, 128, True),  # 32-key tiles, paired causal tiles
    (1, 64, 16, 2048, 2048, 128, True),  # eight waves over 4 GQA heads, 512 work-groups, unpaired
    (2, 64, 16, 4096, 4096, 128, True),  # eight waves over 4 GQA heads, paired causal tiles
    (1, 64, 32, 1500, 1700, 128, True),  # eight waves over 2 GQA heads
    (1, 768, 192, 128, 100, 128, False),  # eight waves, 64-key tiles, one query tile per head
    (1, 64, 16, 1000, 3000, 128, False),  # eight waves, 64-key tiles, 256 work-groups
    (1, 8, 8, 1000, 1000, 64, True),     # direct-to-LDS, D = 64
    (1, 4, 2, 600, 777, 320, True),      # wide-head kernel, 64-key tiles
    (1, 4, 2, 600, 777, 512, False),     # wide-head kernel, 32-key tiles
    (1, 4, 4, 500, 650, 768, False),     # split-D, four waves
    (1, 4, 2, 300, 411, 416, True),      # split-D, four waves, D + 32 layout
    (1, 4, 2, 500, 650, 1024, True),     # split-D, eight waves
    (1, 4, 2, 300, 411, 96, True),       # generic tiled kernel
]


@pytest.mark.parametrize("case", BF16, ids=lambda c: "B{}_Hq{}_Hkv{}_Nq{}_Nkv{}_D{}_{}".format(
    *c[:6], "causal" if c[6] else "full"))
def test_bf16_repeat_launches_bitwise(case):
    B, Hq, Hkv, Nq, Nkv, D, causal = case
    note(f"determinism bf16 {case}")
    w = Workload("det", B, Hq, Hkv, Nq, Nkv, D, causal, "bf16", value_scale=0.5 if D > 256 else 1.0, seed=D)
    q, k, v = (t.cuda() for t in make_inputs(w))
    twice(lambda: A.fwd(q, k, v, causal=causal, scale=w.scale))


def _fp8(case):
    B, Hq, Hkv, Nq, Nkv, D, causal = case
    w = Workload("det8", B, Hq, Hkv, Nq, Nkv, D, causal, "fp8", seed=D + 1, outlier_frac=0.01)
    q8, k8, v8, desc = make_inputs(w)
    dev = torch.device("cuda:0")
    ds = [torch.tensor([float(x)], dtype=torch.float32, device=dev) for x in desc]
    return w, q8.to(dev), k8.to(dev), v8.to(dev), ds


FP8 = [
    (1, 24, 24, 1500, 1500, 128, False),
    (1, 64, 16, 1000, 2000, 128, False),   # eight waves per work-group
    (1, 8, 2, 700, 901, 128, True),
    (1, 4, 2, 500, 600, 256, True),
]


@pytest.mark.parametrize("case", FP8, ids=lambda c: "B{}_Hq{}_Hkv{}_Nq{}_Nkv{}_D{}_{}".format(
    *c[:6], "causal" if c[6] else "full"))
def test_fp8_repeat_launches_bitwise(case):
    note(f"determinism e4m3 {case}")
    w, q, k, v, ds = _fp8(case)
    twice(lambda: A.fwd_fp8(q, k, v, *ds, causal=w.causal, scale=w.scale))


@pytest.mark.parametrize("lean", [False, True], ids=["e4m3_p", "lean_p"])
def test_fp8_probabilities_repeat_launches_bitwise(lean):
    note(f"determinism e4m3 probabilities lean={lean}")
    w, q, k, v, ds = _fp8((1, 32, 8, 2048, 2048, 128, True))
    twice(lambda: A.fwd_fp8_p(q, k, v, *ds, causal=True, scale=w.scale, lean=lean))


def test_fp8_block_descales_repeat_launches_bitwise():
    note("determinism e4m3 block descales")
    w, q, k, v, ds = _fp8((1, 8, 2, 700, 901, 128, True))
    dev = q.device
    bq, bk, bv = (torch.from_numpy(t).to(dev) for t in block_descales(w, seed=1))
    twice(lambda: A.fwd_fp8_blocks(q, k, v, bq, bk, bv, causal=True, scale=w.scale))
