"""Decoding of OCP 8-bit floating point E4M3FN codes to float64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The fp8 path takes per-tensor e4m3 codes plus one descale per tensor (ZYFA
article, section "Getting started with ZYFA": FP8 calls take one descale per
tensor, read from GPU memory).  The oracle runs the plain fp64 definition on
the values the codes stand for, descale * decode(code).  This module turns
codes into exact values, written from the OCP 8-bit floating point
specification (E4M3 with the "FN" encoding):

    bit 7 sign, bits 6..3 exponent e (bias 7), bits 2..0 mantissa f
    e == 0          : subnormal, value = (-1)^s * (f / 8) * 2^(1 - 7)
    e in 1..15      : normal,    value = (-1)^s * (1 + f / 8) * 2^(e - 7)
    e == 15, f == 7 : NaN (the only non-finite code; there is no infinity)

so the largest finite magnitude is 1.75 * 2^8 = 448.
"""
import numpy as np

E4M3FN_MAX = 448.0


def e4m3fn_decode(codes):
    """Exact float64 values of E4M3FN codes (array of uint8, any shape)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    f = (c & 0x7).astype(np.float64)
    sub = (f / 8.0) * 2.0 ** (1 - 7)
    nor = (1.0 + f / 8.0) * np.exp2((e - 7).astype(np.float64))
    val = sign * np.where(e == 0, sub, nor)
    return np.where((e == 15) & ((c & 0x7) == 7), np.nan, val)
