"""Inputs whose scores rise along the key axis, so that the kernels' online
softmax meets a new row maximum on (almost) every key tile: the path that
rescales O and l, and the path that keeps probabilities formed with a stale
maximum.  Plain input construction (torch CPU ops), no attention arithmetic.
"""
import math

import torch


def growing_e4m3(B, H, Hkv, Nq, Nkv, D, gain, seed):
    """e4m3 codes whose scores grow along the key axis by about ``gain``
    (natural units) per key: Q and K codes of N(0, 2^2) values with descale
    1/2 (so the real values are about N(0, 1)), V codes of N(0, 1) values
    with descale 1/4; channel 0 holds the code 4 in every query and about
    a * j in key j (rounded to e4m3, so a non-decreasing staircase), a =
    gain / (scale dq dk 4), capped at the largest finite code 448."""
    g = torch.Generator().manual_seed(seed)
    q = (torch.randn(B, H, Nq, D, generator=g) * 2).clamp(-448, 448)
    k = (torch.randn(B, Hkv, Nkv, D, generator=g) * 2).clamp(-448, 448)
    v = (torch.randn(B, Hkv, Nkv, D, generator=g) * 4).clamp(-448, 448)
    dq, dk, dv = 0.5, 0.5, 0.25
    a = gain / ((1.0 / math.sqrt(D)) * dq * dk * 4.0)
    q[..., 0] = 4.0
    k[..., 0] = (a * torch.arange(Nkv, dtype=torch.float32)).clamp(max=448.0)
    cast = lambda t: t.to(torch.float8_e4m3fn)
    return cast(q), cast(k), cast(v), (dq, dk, dv)
