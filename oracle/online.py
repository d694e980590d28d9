"""The online-softmax recurrence over key blocks, float64, CPU.

TEST INFRASTRUCTURE ONLY (see the package docstring).

This is the algorithm the tiled GPU kernel runs, written out in the order and
notation of the FlashAttention v1/v2/v3/v4 blog post, section "El truco que
hizo posible todo: online softmax": a running max m and running sum l are
kept; for each new block of scores with block max m_new,

    m'  = max(m, m_new)
    l'  = e^{m - m'} * l + sum_{j in block} e^{x_j - m'}
    O'  = e^{m - m'} * O + sum_{j in block} e^{x_j - m'} v_j

and dividing by the final l gives the softmax exactly.  Keeping O
unnormalised until the end is the FA2 change described in the section
"FA2 — paralelizar en serie" (fewer non-matmul operations).

The optional lazy threshold ``tau`` follows the ZYFA article, section "The
details that make it production-grade": the running max is only moved (and O,
l rescaled) when the block max exceeds it by more than tau, measured in base-2
units of the score.  With a stale max the probabilities may exceed 1 (by at
most 2**tau), but O/l and m + ln(l) are unchanged, so the result stays exact.

It exists only so that tests can show, on the CPU and before any GPU code,
that the blockwise recurrence reproduces the plain definition in
``oracle.attention`` (to ~1e-12) for arbitrary block sizes and thresholds.
"""
import math

import numpy as np

from .exact import visible_mask


def online_attention_head(q, k, v, scale, causal=False, block_sizes=(64,), tau=0.0):
    """One (batch, head) of attention by the online recurrence over key blocks.

    ``block_sizes`` is cycled to cut the Nkv keys into consecutive blocks.
    ``tau`` >= 0 is the lazy-rescale threshold in base-2 units.
    Returns (O, LSE) like ``oracle.exact.attention_head``.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    Nq, Nkv = q.shape[0], k.shape[0]
    vis_all = visible_mask(Nq, Nkv, causal)
    tau_nat = float(tau) * math.log(2.0)

    m = np.full(Nq, -np.inf)
    l = np.zeros(Nq)
    O = np.zeros((Nq, v.shape[1]))
    start, bi = 0, 0
    while start < Nkv:
        bs = int(block_sizes[bi % len(block_sizes)])
        bi += 1
        stop = min(Nkv, start + bs)
        x = (q @ k[start:stop].T) * np.float64(scale)
        vis = vis_all[:, start:stop]
        x = np.where(vis, x, -np.inf)
        m_blk = x.max(axis=1, initial=-np.inf)
        # Move the running max only when the block max exceeds it by > tau.
        move = m_blk > m + tau_nat
        m_new = np.where(move, np.maximum(m, m_blk), m)
        finite = np.isfinite(m_new)
        ref = np.where(finite, m_new, 0.0)
        alpha = np.where(np.isfinite(m), np.exp(m - ref), 0.0)
        p = np.where(vis, np.exp(x - ref[:, None]), 0.0)
        l = alpha * l + p.sum(axis=1)
        O = alpha[:, None] * O + p @ v[start:stop]
        m = m_new
        start = stop
    has = l > 0
    O = np.where(has[:, None], O / np.where(has, l, 1.0)[:, None], 0.0)
    lse = np.where(has, m + np.log(np.where(has, l, 1.0)), -np.inf)
    return O, lse
