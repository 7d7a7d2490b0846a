"""fp64 CPU oracle for the attention forward's score variants: sliding
window, ALiBi and softcap.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module.  The HIP
library never routes through it and shares no code with it.

The code-reading page lists these three as compile-time switches next to
causal masking ("FlashAttention — IO 感知的精确注意力 kernel", §1 capability
table) and gives no formulas.  The readings taken, for query i and key j of a
sequence with delta = Lk - Lq (the same bottom-right alignment as causal):

  * x_ij = scale <q_i, k_j>
  * softcap c > 0: x_ij = c tanh(x_ij / c)           (applied to the scaled score)
  * ALiBi slope m_h: x_ij = x_ij - m_h |i + delta - j| (after the softcap)
  * window (left, right), a negative bound open: key j is admissible when
        i + delta - left <= j <= i + delta + right,
    and, when causal, also j <= i + delta.
  * O_i and LSE_i are the plain definition of ``oracle.exact`` over the
    admissible keys with scores x_ij; no admissible key gives O = 0, LSE = -inf.
"""
from __future__ import annotations

import numpy as np

from .exact import _group, kv_head, softmax_rows, to_f64


def variant_scores(qh, kh, scale: float, softcap: float, slope: float) -> np.ndarray:
    """x [lq, lk] of one (sequence, head) after the softcap and the ALiBi bias."""
    lq, lk = qh.shape[0], kh.shape[0]
    x = scale * (qh @ kh.T)
    if softcap > 0:
        x = softcap * np.tanh(x / softcap)
    if slope:
        dist = np.abs(np.arange(lq)[:, None] + (lk - lq) - np.arange(lk)[None, :])
        x = x - slope * dist
    return x


def window_mask(lq: int, lk: int, causal: bool, left: int, right: int) -> np.ndarray:
    """Admissible (i, j) pairs [lq, lk]."""
    i = np.arange(lq)[:, None] + (lk - lq)
    j = np.arange(lk)[None, :]
    m = np.ones((lq, lk), dtype=bool)
    if left >= 0:
        m &= j >= i - left
    if right >= 0:
        m &= j <= i + right
    if causal:
        m &= j <= i
    return m


def head_attention_ext(qh, kh, vh, scale, causal, left, right, softcap, slope):
    """(O [lq, d], LSE [lq]) of one (sequence, head)."""
    lq, lk = qh.shape[0], kh.shape[0]
    x = variant_scores(qh, kh, scale, softcap, slope)
    p, m, l = softmax_rows(x, window_mask(lq, lk, causal, left, right))
    ok = l > 0
    out = np.zeros((lq, vh.shape[1]))
    out[ok] = (p[ok] @ vh) / l[ok][:, None]
    lse = np.full(lq, -np.inf)
    lse[ok] = m[ok] + np.log(l[ok])
    return out, lse


def _slope(alibi, b: int, h: int) -> float:
    if alibi is None:
        return 0.0
    a = np.asarray(alibi, np.float64)
    return float(a[h] if a.ndim == 1 else a[b, h])


def attention_ext(q, k, v, scale: float, causal: bool = False, window=(-1, -1),
                  softcap: float = 0.0, alibi=None):
    """Fixed-length batch: q [B, Nq, Hq, d], k/v [B, Nk, Hkv, d]; alibi slopes
    [Hq] or [B, Hq].  Returns (O [B, Nq, Hq, d], LSE [B, Nq, Hq])."""
    q, k, v = to_f64(q), to_f64(k), to_f64(v)
    bsz, nq, hq, d = q.shape
    g = _group(hq, k.shape[2])
    out = np.zeros((bsz, nq, hq, v.shape[3]))
    lse = np.full((bsz, nq, hq), -np.inf)
    for b in range(bsz):
        for h in range(hq):
            kh = kv_head(h, g)
            out[b, :, h], lse[b, :, h] = head_attention_ext(
                q[b, :, h], k[b, :, kh], v[b, :, kh], scale, causal, window[0], window[1],
                softcap, _slope(alibi, b, h))
    return out, lse


def attention_ext_varlen(q, k, v, cu_q, cu_k, scale: float, causal: bool = False,
                         window=(-1, -1), softcap: float = 0.0, alibi=None):
    """Packed sequences: q [Tq, Hq, d], k/v [Tk, Hkv, d]."""
    q, k, v = to_f64(q), to_f64(k), to_f64(v)
    hq = q.shape[1]
    g = _group(hq, k.shape[1])
    out = np.zeros((q.shape[0], hq, v.shape[2]))
    lse = np.full((q.shape[0], hq), -np.inf)
    for s in range(len(cu_q) - 1):
        qa, qb, ka, kb = int(cu_q[s]), int(cu_q[s + 1]), int(cu_k[s]), int(cu_k[s + 1])
        for h in range(hq):
            kh = kv_head(h, g)
            out[qa:qb, h], lse[qa:qb, h] = head_attention_ext(
                q[qa:qb, h], k[ka:kb, kh], v[ka:kb, kh], scale, causal, window[0], window[1],
                softcap, _slope(alibi, s, h))
    return out, lse
