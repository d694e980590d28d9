"""The polynomial base-2 exponential of the inexact-softmax variant.

TEST INFRASTRUCTURE ONLY (see the package docstring).

FlashAttention v1/v2/v3/v4 blog post, table of ideas: FA4 computes
exponentials with a polynomial instead of the special-function unit.  Reading
taken (the post gives no polynomial): 2^y = 2^j p(f) with j = floor(y),
f = y - j in [0, 1) and the cubic p(f) = 1 + a f + b f^2 + c f^3 whose float32
coefficients were fitted to minimise the largest relative error on [0, 1);
y at or below -150 gives 0 (below float32's smallest subnormal, where the
device's result underflows).  Written in float64 from the float32
coefficients.
"""
import numpy as np

COEFFS = (np.float32(0.69511634), np.float32(0.22764705), np.float32(0.07706515))


def poly_exp2(y):
    """2^y by the cubic above (float64 arithmetic on the float32 coefficients)."""
    y0 = np.asarray(y, dtype=np.float64)
    y = np.maximum(y0, -200.0)
    j = np.floor(y)
    f = y - j
    a, b, c = (float(x) for x in COEFFS)
    p = 1.0 + f * (a + f * (b + f * c))
    return np.where(y0 <= -150.0, 0.0, np.ldexp(p, j.astype(np.int64)))
