"""Attention over one range of the keys, and the merge of such partial
results by their log-sum-exp, in float64 on the CPU.

TEST INFRASTRUCTURE ONLY (see the package docstring): nothing on the product
path may import this module.

ZYFA article, section "The details that make it production-grade": results
computed over different key ranges have to merge consistently, which is what
chunked prefill needs; the same merge finishes a split over keys (split-KV)
and ring attention.  What is computed:

  * attention_range: the plain definition of exact attention (module
    ``exact``) with the visible keys further restricted to the range
    kv_begin <= j < kv_end of the full key sequence.  The causal mask keeps
    the alignment of the whole problem (key j visible to query i iff
    j <= i + Nkv - Nq, j the absolute key index), so a range that ends before
    a row's first visible key leaves that row empty: O = 0, LSE = -inf.
  * merge: for partial results (O_p, LSE_p) over disjoint key ranges,
        LSE = ln sum_p exp(LSE_p),    O = sum_p exp(LSE_p - LSE) O_p,
    which follows from l = sum_p l_p and O = sum_p l_p O_p / l with
    l_p = exp(LSE_p) (the unnormalised row sums of each range share the
    scores' scale).  Rows that are empty in every part stay O = 0,
    LSE = -inf.
"""
import numpy as np

from .exact import kv_head_of, masked_softmax_pv, visible_mask


def key_range_mask(Nq, Nkv, causal, kv_begin, kv_end, rows=None):
    """Boolean (len(rows), Nkv): key j visible to row i and kv_begin <= j < kv_end."""
    vis = visible_mask(Nq, Nkv, causal, rows)
    j = np.arange(Nkv, dtype=np.int64)[None, :]
    return vis & (j >= kv_begin) & (j < kv_end)


def attention_range_head(q, k, v, scale, causal, kv_begin, kv_end, rows=None):
    """Exact attention of one (batch, query head) over keys [kv_begin, kv_end)
    of its full key sequence; float64 (O, LSE) as ``exact.attention_head``."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    Nq, Nkv = q.shape[0], k.shape[0]
    if rows is None:
        rows = np.arange(Nq)
    rows = np.asarray(rows, dtype=np.int64)
    S = (q[rows] @ k.T) * np.float64(scale)
    return masked_softmax_pv(S, key_range_mask(Nq, Nkv, causal, kv_begin, kv_end, rows), v)


def attention_range(q, k, v, scale, causal, kv_begin, kv_end):
    """Whole (B, H, N, D) problem restricted to keys [kv_begin, kv_end)."""
    q = np.asarray(q, dtype=np.float64)
    B, Hq, Nq, _ = q.shape
    Hkv = k.shape[1]
    O = np.empty(q.shape[:3] + (v.shape[3],), dtype=np.float64)
    lse = np.empty((B, Hq, Nq), dtype=np.float64)
    for b in range(B):
        for hq in range(Hq):
            hk = kv_head_of(hq, Hq, Hkv)
            O[b, hq], lse[b, hq] = attention_range_head(q[b, hq], k[b, hk], v[b, hk], scale, causal,
                                                        kv_begin, kv_end)
    return O, lse


def merge(O_parts, LSE_parts):
    """Merge partial results stacked on axis 0: O_parts (P, ..., D),
    LSE_parts (P, ...).  Returns (O, LSE) in float64."""
    O_parts = np.asarray(O_parts, dtype=np.float64)
    LSE_parts = np.asarray(LSE_parts, dtype=np.float64)
    m = LSE_parts.max(axis=0)
    any_part = np.isfinite(m)
    m_safe = np.where(any_part, m, 0.0)
    w = np.exp(LSE_parts - m_safe[None])                 # exp(-inf) = 0 for empty parts
    tot = w.sum(axis=0)
    tot_safe = np.where(any_part, tot, 1.0)
    lse = np.where(any_part, m_safe + np.log(tot_safe), -np.inf)
    O = (w[..., None] * O_parts).sum(axis=0) / tot_safe[..., None]
    O = np.where(any_part[..., None], O, 0.0)
    return O, lse
