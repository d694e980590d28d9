"""Gradients of exact attention, in float64 on the CPU: the plain chain rule
through the forward definition of ``oracle.exact``.

TEST INFRASTRUCTURE ONLY (see the package docstring).

FlashAttention summary page, method paragraph: the backward pass recomputes
S = Q K^T instead of storing it; FlashAttention v1/v2/v3/v4 blog post,
section "FA1 — el cambio de orden de las operaciones": the backward pass
keeps only the softmax statistics and recomputes S block by block from Q, K
and those statistics; FFPA README feature table: forward and backward.  The
pages give no gradient formulas, so this module writes out the derivative of
the forward definition (for one batch b and query head hq, KV head hk):

    s_ij = scale * q_i . k_j,   p_ij = softmax over visible j of s_ij
                                (0 where j is not visible, and for a row that
                                sees no key)
    O_i  = sum_j p_ij v_j

    dV_j  = sum_i p_ij dO_i                      (dV = P^T dO)
    dp_ij = dO_i . v_j                           (dP = dO V^T)
    delta_i = sum_j p_ij dp_ij                   (the softmax Jacobian's
                                                  row term)
    ds_ij = p_ij (dp_ij - delta_i)               (dS, the gradient w.r.t. the
                                                  scaled scores)
    dq_i  = scale * sum_j ds_ij k_j               (dQ = scale dS K)
    dk_j  = scale * sum_i ds_ij q_i               (dK = scale dS^T Q)

and, for GQA/MQA, dK and dV of a KV head are the sums over the query heads
of its group (each query head reads the same K and V).  Masked entries have
p_ij = 0 and so contribute nothing.  delta_i equals dO_i . O_i (substitute
O_i), the form a kernel computes from the forward output; this module uses
the definition above.

Everything is materialised per head: P is (Nq, Nkv).  No blocking.
"""
import numpy as np

from .exact import kv_head_of, visible_mask


def probabilities_head(q, k, scale, causal=False):
    """P (Nq, Nkv) float64: the softmax of scale * q k^T over visible keys,
    0 elsewhere and on rows that see no key."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    vis = visible_mask(q.shape[0], k.shape[0], causal)
    S = np.where(vis, (q @ k.T) * np.float64(scale), -np.inf)
    any_vis = vis.any(axis=1)
    m = np.where(any_vis, S.max(axis=1, initial=-np.inf), 0.0)
    E = np.where(vis, np.exp(S - m[:, None]), 0.0)
    l = np.where(any_vis, E.sum(axis=1), 1.0)
    return E / l[:, None]


def row_delta(P, dP):
    """delta_i = sum_j p_ij dp_ij."""
    return (P * dP).sum(axis=1)


def attention_backward_head(q, k, v, do, scale, causal=False):
    """dQ (Nq, D), dK (Nkv, D), dV (Nkv, Dv) of one (batch, query head), for
    the upstream gradient ``do`` (Nq, Dv) of O.  float64."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    P = probabilities_head(q, k, scale, causal)
    dv = P.T @ do
    dP = do @ v.T
    dS = P * (dP - row_delta(P, dP)[:, None])
    dq = np.float64(scale) * (dS @ k)
    dk = np.float64(scale) * (dS.T @ q)
    return dq, dk, dv


def attention_backward(q, k, v, do, scale, causal=False):
    """Gradients over a whole (B, H, N, D) problem: dQ (B, Hq, Nq, D),
    dK (B, Hkv, Nkv, D), dV (B, Hkv, Nkv, Dv), float64; dK and dV sum over
    the query heads of each KV head's group."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    B, Hq = q.shape[:2]
    Hkv = k.shape[1]
    dq = np.zeros(q.shape, dtype=np.float64)
    dk = np.zeros(k.shape, dtype=np.float64)
    dv = np.zeros(v.shape, dtype=np.float64)
    for b in range(B):
        for hq in range(Hq):
            hk = kv_head_of(hq, Hq, Hkv)
            g_q, g_k, g_v = attention_backward_head(q[b, hq], k[b, hk], v[b, hk], do[b, hq], scale, causal)
            dq[b, hq] = g_q
            dk[b, hk] += g_k
            dv[b, hk] += g_v
    return dq, dk, dv
