"""Host-side checks of the seeded input generators (no GPU)."""
import numpy as np
import torch

import oracle
from exact_io_aware_attn_amd.inputs import WORKLOADS, Workload, make_inputs, quantize_e4m3


def test_same_seed_same_tensors():
    w = Workload("t", 1, 4, 2, 33, 47, 64, True, "bf16", seed=3)
    a = make_inputs(w)
    b = make_inputs(w)
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    c = make_inputs(w.replace(seed=4))
    assert not torch.equal(a[0], c[0])


def test_shapes_and_dtypes():
    w = Workload("t", 2, 4, 2, 5, 7, 32, False, "f32")
    q, k, v = make_inputs(w)
    assert q.shape == (2, 4, 5, 32) and k.shape == (2, 2, 7, 32) and v.shape == (2, 2, 7, 32)
    assert q.dtype == torch.float32
    q, k, v = make_inputs(w.replace(dtype="bf16"))
    assert q.dtype == torch.bfloat16


def test_fp8_recipe_outliers_and_descales():
    w = Workload("t", 1, 4, 4, 64, 64, 32, False, "fp8", outlier_frac=0.05)
    q8, k8, v8, desc = make_inputs(w)
    assert q8.dtype == torch.float8_e4m3fn and desc.dtype == np.float32
    n_out = round(0.05 * 4 * 32)
    for c, d in zip((q8, k8, v8), desc):
        vals = oracle.e4m3fn_decode(c.view(torch.uint8).numpy()) * float(d)
        assert np.isfinite(vals).all()
        # absmax maps to the largest code
        assert np.abs(c.view(torch.uint8).numpy() & 0x7F).max() == 0x7E
        # outlier columns have ~8x the RMS of the others
        rms = np.sqrt((vals ** 2).mean(axis=(0, 2)))  # (H, D)
        big = np.sort(rms.ravel())[::-1]
        assert big[n_out - 1] > 4 * np.median(rms) and big[n_out] < 2 * np.median(rms)


def test_quantize_round_trip_error():
    x = np.random.default_rng(0).standard_normal((3, 1000)) * 3
    codes, d = quantize_e4m3(x)
    back = oracle.e4m3fn_decode(codes.view(torch.uint8).numpy()) * float(d)
    # e4m3 has 3 mantissa bits: relative error <= 2^-4 for normal values
    normal = np.abs(x) / float(d) >= 2.0 ** -6
    assert np.all(np.abs(back - x)[normal] <= np.abs(x)[normal] * 2.0 ** -4 + 1e-12)


def test_flop_count_convention():
    w = WORKLOADS["prefill_causal_bf16"]
    assert w.visible_pairs == 4096 * 4097 // 2
    assert w.flops == 4 * 4 * 32 * 128 * (4096 * 4097 // 2)
    c = WORKLOADS["gqa_cross_bf16"]
    assert c.visible_pairs == 2048 * 8192
    # causal with Nq > Nkv: the first Nq - Nkv rows see nothing
    t = Workload("t", 1, 1, 1, 10, 4, 32, True, "bf16")
    assert t.visible_pairs == sum(min(4, max(0, i - 6 + 1)) for i in range(10))
