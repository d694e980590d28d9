"""The plain definition of exact attention forward, in float64 on the CPU.

TEST INFRASTRUCTURE ONLY (see the package docstring): nothing on the product
path may import this module.

What is computed, for every batch b, query head hq and query row i
(FlashAttention v1/v2/v3/v4 blog post, section "Por qué standard attention era
el cuello de botella": two matmuls with a softmax between them, S = Q K^T
materialised; same post, section "El truco que hizo posible todo: online
softmax": softmax(x_i) = e^{x_i - m} / sum_j e^{x_j - m} with m the row max;
FlashAttention summary page, method paragraph: the tiled algorithm is exact,
so this plain form is the result it must reproduce):

    hk        = hq // (Hq // Hkv)                       (GQA/MQA head groups)
    s_ij      = scale * sum_d q[b,hq,i,d] * k[b,hk,j,d]
    visible_ij = (not causal) or (j <= i + Nkv - Nq)     (bottom-right causal)
    m_i       = max over visible j of s_ij
    p_ij      = exp(s_ij - m_i) if visible else 0,   l_i = sum_j p_ij
    O_i       = sum_j p_ij * v[b,hk,j,:] / l_i
    LSE_i     = m_i + ln(l_i)                            (natural log)

A row with no visible key (possible only when causal and Nq > Nkv) has
O_i = 0 and LSE_i = -inf.

Readings taken where the pages are silent:
  * GQA groups are contiguous (query head hq uses KV head hq // (Hq/Hkv));
    the FFPA README only states that Hq != Hkv is supported.
  * Causal alignment is bottom-right (key j visible to query i iff
    j <= i + Nkv - Nq).  The FFPA README follows SDPA, the ZYFA article the
    flash-attention-2 argument order; the two agree whenever Nq == Nkv.
  * LSE is the natural log of sum_j exp(s_ij) over visible keys.

No blocking, no online recurrence, no base-2 exponentials: S is built whole
for each (b, hq) with one matrix product, masked, and reduced row by row.
"""
import numpy as np


def kv_head_of(hq, Hq, Hkv):
    """KV head used by query head ``hq`` (contiguous GQA/MQA groups).

    FFPA README feature table (GQA/MQA: Hq != Hkv); ZYFA article, section
    "Who should actually run it" (MHA, GQA and MQA).  Requires Hq % Hkv == 0.
    """
    if Hq % Hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    return hq // (Hq // Hkv)


def visible_mask(Nq, Nkv, causal, rows=None):
    """Boolean (len(rows), Nkv) array: True where key j is visible to row i.

    Causal is bottom-right aligned: j <= i + (Nkv - Nq).  ``rows`` selects
    absolute query row indices (default: all rows).
    """
    if rows is None:
        rows = np.arange(Nq)
    rows = np.asarray(rows, dtype=np.int64)
    j = np.arange(Nkv, dtype=np.int64)[None, :]
    if not causal:
        return np.ones((rows.size, Nkv), dtype=bool)
    return j <= (rows[:, None] + (Nkv - Nq))


def attention_head(q, k, v, scale, causal=False, rows=None):
    """Exact attention for one (batch, query head) in float64.

    q: (Nq, D), k: (Nkv, D), v: (Nkv, Dv) arrays (any float dtype; promoted to
    float64).  ``rows``: optional absolute query-row indices to compute (the
    causal mask uses the absolute index), so sampled rows of a large problem
    cost only their own row of S.

    Returns (O, LSE): O (len(rows), Dv) float64, LSE (len(rows),) float64.
    Follows the blog post's softmax with max subtraction (section "El truco
    que hizo posible todo: online softmax") applied to a fully materialised
    S (section "Por qué standard attention era el cuello de botella").
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    Nq, Nkv = q.shape[0], k.shape[0]
    if rows is None:
        rows = np.arange(Nq)
    rows = np.asarray(rows, dtype=np.int64)
    qs = q[rows]
    S = (qs @ k.T) * np.float64(scale)                  # (R, Nkv), materialised
    return masked_softmax_pv(S, visible_mask(Nq, Nkv, causal, rows), v)


def masked_softmax_pv(S, vis, v):
    """Softmax of each row of S over the entries where ``vis`` is True, times
    v; returns (O, LSE).  A row with no True entry gets O = 0, LSE = -inf.

    The max-subtracted softmax of the blog post (section "El truco que hizo
    posible todo: online softmax"), natural log for the LSE.
    """
    S = np.where(vis, S, -np.inf)
    any_vis = vis.any(axis=1)
    m = np.where(any_vis, S.max(axis=1, initial=-np.inf), 0.0)
    P = np.where(vis, np.exp(S - m[:, None]), 0.0)
    l = P.sum(axis=1)
    O = P @ v
    safe_l = np.where(any_vis, l, 1.0)
    O = np.where(any_vis[:, None], O / safe_l[:, None], 0.0)
    lse = np.where(any_vis, m + np.log(safe_l), -np.inf)
    return O, lse


def attention(q, k, v, scale, causal=False):
    """Exact attention over a whole (B, H, N, D) problem, float64.

    q: (B, Hq, Nq, D); k, v: (B, Hkv, Nkv, D).  Returns O (B, Hq, Nq, D) and
    LSE (B, Hq, Nq), both float64.  Layout follows SDPA (FFPA README, section
    "Quick Start": layout (B, H, N, D)).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, Hq, Nq, _ = q.shape
    Hkv = k.shape[1]
    O = np.empty(q.shape[:3] + (v.shape[3],), dtype=np.float64)
    lse = np.empty((B, Hq, Nq), dtype=np.float64)
    for b in range(B):
        for hq in range(Hq):
            hk = kv_head_of(hq, Hq, Hkv)
            O[b, hq], lse[b, hq] = attention_head(q[b, hq], k[b, hk], v[b, hk], scale, causal)
    return O, lse
