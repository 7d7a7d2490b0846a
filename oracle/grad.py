"""fp64 CPU oracle for the gradients of exact attention.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module.  The HIP
library never routes through it and shares no code with it.

What it computes: for the forward of ``oracle.exact`` (O = softmax(scale Q Kᵀ)
V over the admissible keys) and an upstream gradient dO, the gradients of the
scalar <dO, O> with respect to Q, K and V.  The pages give the backward's
structure, not its formulas: the backward keeps only O and the per-row
logsumexp and recomputes P from them instead of storing it ("FlashAttention
— IO 感知的精确注意力 kernel", §2.3 and §4: the backward recomputes P and
accumulates dK/dV per key block; the blog post's table of FlashAttention 1
engineering lists recomputation in the backward).  The formulas below are
the derivative of the definition, written out with the chain rule:

    P    = row-softmax of S = scale Q Kᵀ (zero outside the mask)
    dV   = Pᵀ dO
    dP   = dO Vᵀ
    dS   = P ∘ (dP − rowsum(P ∘ dP))          (Jacobian of a softmax row)
    dQ   = scale dS K,    dK = scale dSᵀ Q

With grouped heads a key/value head receives the sum of the gradients of
all query heads that read it.  A row with no admissible key has P = 0 and
contributes nothing.
"""
from __future__ import annotations

import numpy as np

from .exact import _group, admissible_mask, kv_head, scores, softmax_rows, to_f64


def probabilities(qh, kh, scale: float, causal: bool) -> np.ndarray:
    """Normalised P [lq, lk] of one (sequence, head), zero outside the mask and
    on rows with no admissible key."""
    lq, lk = qh.shape[0], kh.shape[0]
    mask = admissible_mask(np.arange(lq), lq, lk, causal)
    p, _, l = softmax_rows(scores(qh, kh, scale), mask)
    safe = np.where(l > 0, l, 1.0)
    return np.where((l > 0)[:, None], p / safe[:, None], 0.0)


def value_grad(p, doh):
    """dV = Pᵀ dO."""
    return p.T @ doh


def prob_grad(doh, vh):
    """dP = dO Vᵀ."""
    return doh @ vh.T


def softmax_backward(p, dp):
    """dS = P ∘ (dP − rowsum(P ∘ dP)): the softmax Jacobian applied per row."""
    return p * (dp - (p * dp).sum(axis=1, keepdims=True))


def query_grad(ds, kh, scale: float):
    """dQ = scale dS K."""
    return scale * (ds @ kh)


def key_grad(ds, qh, scale: float):
    """dK = scale dSᵀ Q."""
    return scale * (ds.T @ qh)


def head_attention_grad(qh, kh, vh, doh, scale: float, causal: bool):
    """(dQ [lq, d], dK [lk, d], dV [lk, d]) of one (sequence, head)."""
    p = probabilities(qh, kh, scale, causal)
    ds = softmax_backward(p, prob_grad(doh, vh))
    return query_grad(ds, kh, scale), key_grad(ds, qh, scale), value_grad(p, doh)


def attention_grad(q, k, v, do, scale: float, causal: bool = False):
    """Fixed-length batch: q/do [B, Nq, Hq, d], k/v [B, Nk, Hkv, d].

    Returns (dQ [B, Nq, Hq, d], dK [B, Nk, Hkv, d], dV [B, Nk, Hkv, d]), fp64.
    """
    q, k, v, do = to_f64(q), to_f64(k), to_f64(v), to_f64(do)
    bsz, _, hq, _ = q.shape
    hkv = k.shape[2]
    g = _group(hq, hkv)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(bsz):
        for h in range(hq):
            kh = kv_head(h, g)
            gq, gk, gv = head_attention_grad(q[b, :, h], k[b, :, kh], v[b, :, kh], do[b, :, h],
                                             scale, causal)
            dq[b, :, h] = gq
            dk[b, :, kh] += gk
            dv[b, :, kh] += gv
    return dq, dk, dv


def attention_grad_varlen(q, k, v, do, cu_q, cu_k, scale: float, causal: bool = False):
    """Packed sequences (the layout of ``oracle.exact.attention_varlen``):
    q/do [Tq, Hq, d], k/v [Tk, Hkv, d].  Returns (dQ, dK, dV) in that layout."""
    q, k, v, do = to_f64(q), to_f64(k), to_f64(v), to_f64(do)
    cu_q, cu_k = np.asarray(cu_q, np.int64), np.asarray(cu_k, np.int64)
    hq, hkv = q.shape[1], k.shape[1]
    g = _group(hq, hkv)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for s in range(len(cu_q) - 1):
        qa, qb, ka, kb = cu_q[s], cu_q[s + 1], cu_k[s], cu_k[s + 1]
        for h in range(hq):
            kh = kv_head(h, g)
            gq, gk, gv = head_attention_grad(q[qa:qb, h], k[ka:kb, kh], v[ka:kb, kh],
                                             do[qa:qb, h], scale, causal)
            dq[qa:qb, h] = gq
            dk[ka:kb, kh] += gk
            dv[ka:kb, kh] += gv
    return dq, dk, dv
