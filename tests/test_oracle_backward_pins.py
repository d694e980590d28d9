"""Pins for the oracle's attention gradients (``oracle/backward.py``).

Each ``check_*`` returns True when the oracle's dQ, dK, dV agree with a fact
that does not come from the backward module itself:
  * central finite differences of the forward oracle on tiny problems (the
    gradient is the derivative of the forward definition), causal and not,
    GQA, a row that sees no key;
  * torch's CPU float64 autograd through a plainly written softmax attention
    (a library routine);
  * invariants: the rows of dS sum to zero, so sum_j dK_j = 0 for every head;
    the rows of P sum to one, so sum_j dV_j = sum_i dO_i over rows that see a
    key; dQ_i = 0 for a row that sees no key;
  * closed forms: constant V rows give dQ = dK = 0; a single visible key gives
    dV_0 = sum_i dO_i and dQ = dK = 0; scale 0 gives uniform P, so every dV_j
    is sum_i dO_i / Nkv, and dQ = dK = 0.
``test_backward_planted_mistakes_are_caught`` plants plausible mistakes in the
backward oracle and asserts that some check fails for each.
"""
import numpy as np
import pytest
import torch

import oracle
import oracle.backward as obwd
from oracle import attention

RTOL_FD = 1e-6


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def _problem(seed, B, Hq, Hkv, Nq, Nkv, D):
    rng = np.random.default_rng(seed)
    return (_rand(rng, B, Hq, Nq, D), _rand(rng, B, Hkv, Nkv, D), _rand(rng, B, Hkv, Nkv, D),
            _rand(rng, B, Hq, Nq, D))


def finite_difference_grads(q, k, v, g, scale, causal, h=1e-5):
    """Gradients of L = sum(O * g) by central differences of the forward
    oracle, one input element at a time."""
    def loss(qq, kk, vv):
        O, _ = attention(qq, kk, vv, scale, causal)
        return float((O * g).sum())

    out = []
    for which in range(3):
        args = [q.copy(), k.copy(), v.copy()]
        x = args[which]
        grad = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            x0 = x[idx]
            x[idx] = x0 + h
            lp = loss(*args)
            x[idx] = x0 - h
            lm = loss(*args)
            x[idx] = x0
            grad[idx] = (lp - lm) / (2 * h)
        out.append(grad)
    return out


def _close(a, b, rtol):
    scale = max(1.0, float(np.abs(b).max()))
    return float(np.abs(a - b).max()) <= rtol * scale


def check_finite_differences():
    ok = True
    for seed, (B, Hq, Hkv, Nq, Nkv, D), causal in [
        (0, (1, 2, 1, 3, 5, 4), False),
        (1, (1, 2, 2, 4, 4, 3), True),
        (2, (1, 2, 1, 5, 3, 4), True),     # Nq > Nkv: the first two rows see no key
        (3, (2, 1, 1, 4, 6, 2), True),
    ]:
        q, k, v, g = _problem(seed, B, Hq, Hkv, Nq, Nkv, D)
        scale = 0.7
        dq, dk, dv = oracle.attention_backward(q, k, v, g, scale, causal)
        fq, fk, fv = finite_difference_grads(q, k, v, g, scale, causal)
        ok &= _close(dq, fq, RTOL_FD) and _close(dk, fk, RTOL_FD) and _close(dv, fv, RTOL_FD)
    return ok


def check_torch_autograd():
    """torch float64 autograd through softmax(scale q k^T + mask) v, K and V
    repeated over each GQA group."""
    ok = True
    for seed, (B, Hq, Hkv, Nq, Nkv, D), causal in [
        (4, (2, 4, 2, 37, 53, 16), True),
        (5, (1, 3, 1, 29, 29, 8), False),
        (6, (1, 2, 2, 40, 17, 8), True),
    ]:
        q, k, v, g = _problem(seed, B, Hq, Hkv, Nq, Nkv, D)
        scale = 1.0 / np.sqrt(D)
        tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
        G = Hq // Hkv
        kk = tk.repeat_interleave(G, dim=1)
        vv = tv.repeat_interleave(G, dim=1)
        S = torch.matmul(tq, kk.transpose(-1, -2)) * scale
        if causal:
            i = torch.arange(Nq)[:, None]
            j = torch.arange(Nkv)[None, :]
            vis = j <= i + (Nkv - Nq)
            S = S.masked_fill(~vis, float("-inf"))
        P = torch.softmax(S, dim=-1)
        P = torch.nan_to_num(P, nan=0.0)        # rows with no visible key
        O = torch.matmul(P, vv)
        (O * torch.tensor(g)).sum().backward()
        dq, dk, dv = oracle.attention_backward(q, k, v, g, scale, causal)
        ok &= _close(dq, tq.grad.numpy(), 1e-10) and _close(dk, tk.grad.numpy(), 1e-10) and \
            _close(dv, tv.grad.numpy(), 1e-10)
    return ok


def check_invariants():
    ok = True
    for seed, (B, Hq, Hkv, Nq, Nkv, D), causal in [
        (7, (1, 4, 2, 33, 47, 8), True),
        (8, (2, 2, 1, 50, 20, 8), True),      # rows without keys
        (9, (1, 2, 2, 31, 31, 8), False),
    ]:
        q, k, v, g = _problem(seed, B, Hq, Hkv, Nq, Nkv, D)
        dq, dk, dv = oracle.attention_backward(q, k, v, g, 0.4, causal)
        # sum_j dK_j = 0: a common shift of every key moves each row's scores
        # by a constant, which the softmax ignores
        ok &= np.abs(dk.sum(axis=2)).max() <= 1e-10 * max(1.0, np.abs(dk).max())
        # sum_j dV_j = sum over the group's rows that see a key of dO_i
        G = Hq // Hkv
        seen = oracle.visible_mask(Nq, Nkv, causal).any(axis=1)
        for b in range(B):
            for hk in range(Hkv):
                want = g[b, hk * G:(hk + 1) * G][:, seen].sum(axis=(0, 1))
                ok &= np.allclose(dv[b, hk].sum(axis=0), want, rtol=1e-10, atol=1e-10)
        # rows that see no key have no gradient
        ok &= bool((dq[:, :, ~seen] == 0).all())
    return ok


def check_closed_forms():
    ok = True
    rng = np.random.default_rng(10)
    # constant V rows: O does not depend on P, so dQ = dK = 0
    q, k, _, g = _problem(11, 1, 2, 1, 9, 13, 4)
    v = np.tile(rng.standard_normal(4), (1, 1, 13, 1))
    dq, dk, dv = oracle.attention_backward(q, k, v, g, 0.9, False)
    ok &= np.abs(dq).max() <= 1e-12 and np.abs(dk).max() <= 1e-12
    # a single key: p = 1 for every row, dV_0 = sum_i dO_i, dQ = dK = 0
    q, k, v, g = _problem(12, 1, 3, 1, 7, 1, 5)
    dq, dk, dv = oracle.attention_backward(q, k, v, g, 1.3, False)
    ok &= np.allclose(dv[0, 0, 0], g[0].sum(axis=(0, 1)), rtol=1e-12, atol=1e-12)
    ok &= np.abs(dq).max() <= 1e-12 and np.abs(dk).max() <= 1e-12
    # scale 0: P uniform 1/Nkv, so dV_j = sum_i dO_i / Nkv for every j, and
    # dQ = dK = 0 (the scale multiplies both)
    q, k, v, g = _problem(13, 1, 2, 2, 6, 8, 3)
    dq, dk, dv = oracle.attention_backward(q, k, v, g, 0.0, False)
    ok &= np.allclose(dv, np.broadcast_to(g.sum(axis=2, keepdims=True) / 8, dv.shape), rtol=1e-12, atol=1e-12)
    ok &= np.abs(dq).max() == 0 and np.abs(dk).max() == 0
    return ok


ALL_CHECKS = [check_finite_differences, check_torch_autograd, check_invariants, check_closed_forms]


@pytest.mark.parametrize("check", ALL_CHECKS, ids=lambda c: c.__name__)
def test_backward_oracle_pin(check):
    assert check()


def _mut_delta_unweighted(P, dP):
    return dP.sum(axis=1)


def _mut_delta_dropped(P, dP):
    return np.zeros(P.shape[0])


def _mut_probs_unnormalised(q, k, scale, causal=False):
    P = obwd_orig_probs(q, k, scale, causal)
    return P * P.shape[1]


def _mut_probs_no_scale(q, k, scale, causal=False):
    return obwd_orig_probs(q, k, 1.0, causal)


def _mut_head_no_dq_scale(q, k, v, do, scale, causal=False):
    dq, dk, dv = obwd_orig_head(q, k, v, do, scale, causal)
    return dq / np.float64(scale) if scale else dq, dk, dv


def _mut_head_dk_from_dp(q, k, v, do, scale, causal=False):
    q = np.asarray(q, dtype=np.float64)
    P = obwd.probabilities_head(q, k, scale, causal)
    dq, _, dv = obwd_orig_head(q, k, v, do, scale, causal)
    dP = np.asarray(do) @ np.asarray(v).T
    return dq, np.float64(scale) * ((P * dP).T @ q), dv


def _mut_gqa_overwrite(q, k, v, do, scale, causal=False):
    q = np.asarray(q, dtype=np.float64)
    B, Hq = q.shape[:2]
    Hkv = np.asarray(k).shape[1]
    dq = np.zeros(q.shape)
    dk = np.zeros(np.asarray(k).shape)
    dv = np.zeros(np.asarray(v).shape)
    for b in range(B):
        for hq in range(Hq):
            hk = oracle.kv_head_of(hq, Hq, Hkv)
            dq[b, hq], dk[b, hk], dv[b, hk] = obwd.attention_backward_head(
                q[b, hq], k[b, hk], v[b, hk], do[b, hq], scale, causal)
    return dq, dk, dv


obwd_orig_probs = obwd.probabilities_head
obwd_orig_head = obwd.attention_backward_head

MUTATIONS = {
    "delta_unweighted": (obwd, "row_delta", _mut_delta_unweighted),
    "delta_dropped": (obwd, "row_delta", _mut_delta_dropped),
    "probs_unnormalised": (obwd, "probabilities_head", _mut_probs_unnormalised),
    "probs_scale_dropped": (obwd, "probabilities_head", _mut_probs_no_scale),
    "dq_scale_dropped": (obwd, "attention_backward_head", _mut_head_no_dq_scale),
    "dk_from_dp_not_ds": (obwd, "attention_backward_head", _mut_head_dk_from_dp),
    "gqa_overwrite": (obwd, "attention_backward", _mut_gqa_overwrite),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_backward_planted_mistakes_are_caught(name, monkeypatch):
    mod, attr, fn = MUTATIONS[name]
    monkeypatch.setattr(mod, attr, fn)
    # the checks call oracle.attention_backward, which goes through the module
    monkeypatch.setattr(oracle, "attention_backward", obwd.attention_backward)
    failed = [c.__name__ for c in ALL_CHECKS if not c()]
    assert failed, f"no check caught the planted mistake {name}"
