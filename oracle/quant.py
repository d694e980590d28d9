"""The fp8 input pipeline: rotation of Q and K by a signed Hadamard matrix,
then e4m3 quantisation with one descale per block of rows.

TEST INFRASTRUCTURE ONLY (see the package docstring).

FA blog, section "FA3 — el momento Hopper": FP8 with block quantisation (one
scale per 64 x d tile instead of one per tensor) and incoherent processing
(a pre-multiplication by a random orthogonal Hadamard-based matrix that
spreads outliers before quantising).  ZYFA article, sections "The ZYFA
accuracy work is the sleeper contribution" and "Who should actually run it":
a Hadamard rotation of Q and K before quantisation roughly halves the input
error, and accuracy is measured against fp64 attention.

What is computed (readings where the pages are silent):
  * Rotation R = diag(signs) H_D / sqrt(D), H_D the Sylvester Hadamard matrix
    (entries +-1; H_1 = [1], H_2n = [[H_n, H_n], [H_n, -H_n]]) and signs a
    given vector of +-1 of length D (random numbers drawn outside and passed
    in).  Rows are multiplied on the right, q' = q R.  R is orthogonal, so
    q' k'^T = q k^T: Q and K are rotated, V is not.
  * Blocks: rows [64 i, 64 i + 64) of each (batch, head) slab, the last block
    ragged.  amax = max |x| over a block (after the rotation, in float32);
    descale = amax / 448 and inv = 448 / amax, each rounded to float32; an
    all-zero block has descale 1 and codes 0.
  * code = e4m3fn(x * inv): x the float32 value (the rotated value rounded to
    float32), the product rounded to float32 and then to the nearest e4m3fn
    value, ties to the even code (mantissa bit 0 clear), saturating at +-448.
    These are float32 decisions, the precision the device quantiser takes
    them in.
"""
import numpy as np

from .e4m3 import E4M3FN_MAX, e4m3fn_decode

_POS_CODES = np.arange(0x7F, dtype=np.uint8)          # 0x00 .. 0x7E: 0 .. 448 ascending
_POS_VALUES = e4m3fn_decode(_POS_CODES)


def e4m3fn_encode(x):
    """Nearest e4m3fn code (ties to even code, saturating at 448) of each
    value of x (any float array; exact in float64).  -0 and negatives that
    round to zero keep the sign bit."""
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), E4M3FN_MAX)
    hi = np.clip(np.searchsorted(_POS_VALUES, a, side="left"), 0, 0x7E)
    lo = np.clip(hi - 1, 0, 0x7E)
    d_lo = a - _POS_VALUES[lo]
    d_hi = _POS_VALUES[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & ((hi & 1) == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    return np.where(np.signbit(x), code | 0x80, code).astype(np.uint8)


def hadamard(D):
    """Sylvester Hadamard matrix H_D (float64, entries +-1); D a power of 2."""
    if D < 1 or D & (D - 1):
        raise ValueError("D must be a power of two")
    H = np.ones((1, 1))
    while H.shape[0] < D:
        H = np.block([[H, H], [H, -H]])
    return H


def rotation(signs):
    """R = diag(signs) H_D / sqrt(D) for a +-1 vector of length D."""
    signs = np.asarray(signs, dtype=np.float64)
    D = signs.shape[0]
    return signs[:, None] * hadamard(D) / np.sqrt(D)


def quantize_blocks(x, signs=None, block=64):
    """Block e4m3 quantisation of x (B, H, N, D), optionally rotated first.

    Returns (codes uint8 (B, H, N, D), descales float32 (B, H, ceil(N/block)))."""
    x = np.asarray(x, dtype=np.float64)
    if signs is not None:
        x = x @ rotation(signs)
    x32 = x.astype(np.float32)
    B, H, N, D = x32.shape
    nb = (N + block - 1) // block
    codes = np.empty(x32.shape, dtype=np.uint8)
    desc = np.empty((B, H, nb), dtype=np.float32)
    for i in range(nb):
        blk = x32[:, :, i * block:(i + 1) * block, :]
        amax = np.abs(blk).max(axis=(2, 3)).astype(np.float32)            # exact
        zero = amax == 0
        amax_safe = np.where(zero, np.float32(1.0), amax).astype(np.float32)
        d = np.where(zero, np.float32(1.0), amax_safe / np.float32(E4M3FN_MAX)).astype(np.float32)
        inv = np.where(zero, np.float32(0.0), np.float32(E4M3FN_MAX) / amax_safe).astype(np.float32)
        y = (blk * inv[:, :, None, None]).astype(np.float32)             # float32 product
        codes[:, :, i * block:(i + 1) * block, :] = e4m3fn_encode(y)
        desc[:, :, i] = d
    return codes, desc


def dequantize_blocks(codes, descales, block=64):
    """Exact float64 values decode(code) * descale of each block's rows."""
    v = e4m3fn_decode(codes)
    rows = np.arange(v.shape[2]) // block
    return v * descales.astype(np.float64)[:, :, rows][..., None]
