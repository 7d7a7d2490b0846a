"""fp64 CPU oracle for the exact attention forward.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module.  The HIP
library never routes through it and shares no code with it.

What it computes is the plain definition of scaled dot-product attention
("推理优化 | FlashAttention 1-4 详解", §原算法：标准 Attention 与显存瓶颈, the
three-step S/P/O definition; "FlashAttention — IO 感知的精确注意力 kernel", §1,
which states the fused kernel returns softmax(Q Kᵀ·scale)·V exactly):

    s_ij = scale * <q_i, k_j>                 over admissible keys j
    m_i  = max_j s_ij,  p_ij = exp(s_ij - m_i) (two-pass safe softmax, §Online
           Softmax 数学推导 of the first page, first display)
    l_i  = sum_j p_ij
    O_i  = sum_j (p_ij / l_i) v_j,   LSE_i = m_i + ln l_i

Readings (where the pages leave a step open):
  * scale multiplies Q Kᵀ (the first page's PyTorch listing omits it; its
    formulas keep it).
  * LSE is the natural-log logsumexp of the scaled scores (third page, §2.3
    step 5 names the logsumexp as the second output).
  * causal masks are bottom-right aligned: key j is admissible for query i when
    j <= i + Lk - Lq (the plain lower triangle when Lq == Lk, and "all cached
    keys" for a single decode query, the KV-cache call of the third page, §1).
  * GQA maps query head h to key/value head h // (Hq / Hkv) (third page, §1
    capability table: Hkv must divide Hq).
  * A row with no admissible key has O = 0 and LSE = -inf.

Everything is materialised (S and P per sequence and head, in row chunks), in
float64, with numpy only.  ``tiled_online_attention`` is a second, independent
algorithm (the online-softmax recurrence) used only to pin this one.
"""
from __future__ import annotations

import numpy as np

ROW_CHUNK = 1024


# --------------------------------------------------------------------------
# input decoding
# --------------------------------------------------------------------------
def to_f64(x) -> np.ndarray:
    """bfloat16 bit patterns (uint16) or any float array -> float64 (exact)."""
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return x.astype(np.float64)


# --------------------------------------------------------------------------
# building blocks of the definition
# --------------------------------------------------------------------------
def admissible_mask(row_ids: np.ndarray, lq: int, lk: int, causal: bool) -> np.ndarray:
    """Boolean [len(row_ids), lk]: key j admissible for query row i."""
    j = np.arange(lk)[None, :]
    if not causal:
        return np.ones((len(row_ids), lk), dtype=bool)
    return j <= (np.asarray(row_ids)[:, None] + (lk - lq))


def scores(qh: np.ndarray, kh: np.ndarray, scale: float) -> np.ndarray:
    """S = scale * Q Kᵀ for one head: qh [r, d], kh [lk, d] -> [r, lk]."""
    return scale * (qh @ kh.T)


def kv_head(h: int, group: int) -> int:
    """Key/value head serving query head h when ``group`` query heads share one."""
    return h // group


def weighted_values(p: np.ndarray, vh: np.ndarray, l: np.ndarray) -> np.ndarray:
    """Normalised output rows: (P V) / l for rows with l > 0."""
    return (p @ vh) / l[:, None]


def softmax_rows(s: np.ndarray, mask: np.ndarray):
    """Two-pass safe softmax over admissible entries of each row.

    Returns (P, m, l): P [r, lk] with zeros outside the mask, row max m and
    row sum l of exp(s - m).  Rows without admissible keys get m = -inf, l = 0.
    """
    s = np.where(mask, s, -np.inf)
    m = s.max(axis=1) if s.shape[1] else np.full(s.shape[0], -np.inf)
    has = np.isfinite(m)
    shift = np.where(has, m, 0.0)
    p = np.where(mask, np.exp(s - shift[:, None]), 0.0)
    l = p.sum(axis=1)
    return p, m, l


def head_attention(qh, kh, vh, scale, causal, row_ids=None, lq=None):
    """Attention for one (sequence, head): qh [r, d] (rows ``row_ids`` of a
    sequence of length ``lq``), kh/vh [lk, d].  Returns (O [r, d], LSE [r])."""
    r, d = qh.shape
    lk = kh.shape[0]
    lq = r if lq is None else lq
    row_ids = np.arange(r) if row_ids is None else np.asarray(row_ids)
    out = np.zeros((r, vh.shape[1]), np.float64)
    lse = np.full(r, -np.inf, np.float64)
    for c0 in range(0, r, ROW_CHUNK):
        c1 = min(r, c0 + ROW_CHUNK)
        mask = admissible_mask(row_ids[c0:c1], lq, lk, causal)
        p, m, l = softmax_rows(scores(qh[c0:c1], kh, scale), mask)
        ok = l > 0
        out[c0:c1][ok] = weighted_values(p[ok], vh, l[ok])
        lse[c0:c1][ok] = m[ok] + np.log(l[ok])
    return out, lse


def _group(hq: int, hkv: int) -> int:
    if hkv <= 0 or hq % hkv:
        raise ValueError("heads_kv must divide heads_q")
    return hq // hkv


# --------------------------------------------------------------------------
# public entry points
# --------------------------------------------------------------------------
def attention(q, k, v, scale: float, causal: bool = False):
    """Fixed-length batch: q [B, Nq, Hq, d], k/v [B, Nk, Hkv, d].

    Returns (O [B, Nq, Hq, d] float64, LSE [B, Nq, Hq] float64).
    """
    q, k, v = to_f64(q), to_f64(k), to_f64(v)
    bsz, nq, hq, d = q.shape
    hkv = k.shape[2]
    g = _group(hq, hkv)
    out = np.zeros((bsz, nq, hq, v.shape[3]))
    lse = np.full((bsz, nq, hq), -np.inf)
    for b in range(bsz):
        for h in range(hq):
            kh = kv_head(h, g)
            o_bh, l_bh = head_attention(q[b, :, h], k[b, :, kh], v[b, :, kh],
                                        scale, causal)
            out[b, :, h] = o_bh
            lse[b, :, h] = l_bh
    return out, lse


def attention_varlen(q, k, v, cu_q, cu_k, scale: float, causal: bool = False):
    """Packed sequences: q [Tq, Hq, d], k/v [Tk, Hkv, d]; sequence s owns rows
    [cu_q[s], cu_q[s+1]) of q and [cu_k[s], cu_k[s+1]) of k/v (third page, §1:
    variable-length batches packed through cumulative sequence offsets).

    Returns (O [Tq, Hq, d], LSE [Tq, Hq]).
    """
    q, k, v = to_f64(q), to_f64(k), to_f64(v)
    cu_q, cu_k = np.asarray(cu_q, np.int64), np.asarray(cu_k, np.int64)
    hq, hkv = q.shape[1], k.shape[1]
    g = _group(hq, hkv)
    out = np.zeros((q.shape[0], hq, v.shape[2]))
    lse = np.full((q.shape[0], hq), -np.inf)
    for s in range(len(cu_q) - 1):
        qa, qb, ka, kb = cu_q[s], cu_q[s + 1], cu_k[s], cu_k[s + 1]
        for h in range(hq):
            kh = kv_head(h, g)
            o_sh, l_sh = head_attention(q[qa:qb, h], k[ka:kb, kh], v[ka:kb, kh],
                                        scale, causal)
            out[qa:qb, h] = o_sh
            lse[qa:qb, h] = l_sh
    return out, lse


def attention_rows(q, k, v, rows, scale: float, causal: bool, cu_q=None, cu_k=None):
    """Selected output rows only, computed one by one from the definition.

    ``rows`` is an iterable of (b, i, h): sequence b, query position i within it,
    query head h.  Works for fixed layout (cu_q is None) and packed layout.
    Inputs are widened slice by slice, so full-size workloads fit in memory.
    Returns (O [n, d], LSE [n]).
    """
    q, k, v = np.asarray(q), np.asarray(k), np.asarray(v)
    packed = cu_q is not None
    hq = q.shape[-2]
    hkv = k.shape[-2]
    g = _group(hq, hkv)
    if packed:
        cu_q = np.asarray(cu_q, np.int64)
        cu_k = cu_q if cu_k is None else np.asarray(cu_k, np.int64)
    kv_cache = {}
    outs, lses = [], []
    for (b, i, h) in rows:
        kvh = kv_head(h, g)
        if (b, kvh) not in kv_cache:
            if packed:
                sl = slice(int(cu_k[b]), int(cu_k[b + 1]))
                kv_cache[(b, kvh)] = (to_f64(k[sl, kvh]), to_f64(v[sl, kvh]))
            else:
                kv_cache[(b, kvh)] = (to_f64(k[b, :, kvh]), to_f64(v[b, :, kvh]))
        kh, vh = kv_cache[(b, kvh)]
        if packed:
            lq = int(cu_q[b + 1] - cu_q[b])
            qi = to_f64(q[cu_q[b] + i, h])[None, :]
        else:
            lq = q.shape[1]
            qi = to_f64(q[b, i, h])[None, :]
        o, l = head_attention(qi, kh, vh, scale, causal, row_ids=[i], lq=lq)
        outs.append(o[0])
        lses.append(l[0])
    return np.array(outs), np.array(lses)


def decode(q, k_cache, v_cache, cache_seqlens, scale: float, batches=None):
    """Single-query decode against a KV cache: q [B, Hq, d], caches
    [B, Ncache, Hkv, d], sequence b uses cache rows [0, cache_seqlens[b]) (third
    page, §1: the KV-cache entry point used at decode time).  One query per
    sequence sees every cached key (bottom-right causal with Lq = 1).

    ``batches`` optionally restricts the work to some sequences (others stay
    zero / -inf).  Returns (O [B, Hq, d], LSE [B, Hq]).
    """
    q = to_f64(q)
    bsz, hq, d = q.shape
    hkv = k_cache.shape[2]
    g = _group(hq, hkv)
    out = np.zeros((bsz, hq, v_cache.shape[3]))
    lse = np.full((bsz, hq), -np.inf)
    for b in (range(bsz) if batches is None else batches):
        n = int(cache_seqlens[b])
        kb = to_f64(k_cache[b, :n])
        vb = to_f64(v_cache[b, :n])
        for h in range(hq):
            kh = kv_head(h, g)
            o, l = head_attention(q[b, h][None, :], kb[:, kh], vb[:, kh], scale, causal=False)
            out[b, h] = o[0]
            lse[b, h] = l[0]
    return out, lse


def merge_partials(o_parts, lse_parts):
    """LSE-weighted merge of partial results over disjoint key subsets.

    o_parts [..., S, d] are each part's normalised output, lse_parts [..., S]
    each part's logsumexp (-inf for an empty part).  Follows the block merge of
    the lecture notes ("FlashAttention" notes on the PKU lecture, §6: keep only
    the running max, sum and output per row), written with logsumexps:
        LSE = M + ln sum_s exp(LSE_s - M),  M = max_s LSE_s
        O   = sum_s exp(LSE_s - LSE) * O_s
    All parts empty gives O = 0 and LSE = -inf.
    """
    o_parts = np.asarray(o_parts, np.float64)
    lse_parts = np.asarray(lse_parts, np.float64)
    m = lse_parts.max(axis=-1)
    has = np.isfinite(m)
    msafe = np.where(has, m, 0.0)
    w = np.where(np.isfinite(lse_parts), np.exp(lse_parts - msafe[..., None]), 0.0)
    tot = w.sum(axis=-1)
    lse = np.where(has, msafe + np.log(np.where(has, tot, 1.0)), -np.inf)
    wn = np.where(has[..., None], w / np.where(has, tot, 1.0)[..., None], 0.0)
    o_clean = np.where(np.isfinite(lse_parts)[..., None], o_parts, 0.0)
    out = (wn[..., None] * o_clean).sum(axis=-2)
    return out, lse


def tiled_online_attention(qh, kh, vh, scale: float, br: int, bc: int, causal: bool = False):
    """The online-softmax recomputation, for pinning ``head_attention`` only.

    Follows the tiled algorithm of the first page (§Online Softmax 数学推导 update
    equations and the §PyTorch 实现 description): for each block of ``br`` query
    rows keep a running max m, running sum l and unnormalised output O; for
    each block of ``bc`` keys take m_new = max(m, rowmax S), P = exp(S - m_new),
    l = exp(m - m_new) l + rowsum P, O = exp(m - m_new) O + P V; finally O / l.
    The scale is applied to S (the listing on that page leaves it out).
    """
    qh, kh, vh = to_f64(qh), to_f64(kh), to_f64(vh)
    n, d = qh.shape
    lk = kh.shape[0]
    out = np.zeros((n, vh.shape[1]))
    lse = np.full(n, -np.inf)
    for i0 in range(0, n, br):
        i1 = min(n, i0 + br)
        rows = np.arange(i0, i1)
        o = np.zeros((i1 - i0, vh.shape[1]))
        m = np.full(i1 - i0, -np.inf)
        l = np.zeros(i1 - i0)
        for j0 in range(0, lk, bc):
            j1 = min(lk, j0 + bc)
            s = scale * (qh[i0:i1] @ kh[j0:j1].T)
            if causal:
                allowed = np.arange(j0, j1)[None, :] <= rows[:, None] + (lk - n)
                s = np.where(allowed, s, -np.inf)
            m_new = np.maximum(m, s.max(axis=1))
            fin = np.isfinite(m_new)
            sub = np.where(fin, m_new, 0.0)
            p = np.exp(s - sub[:, None])
            corr = np.where(np.isfinite(m), np.exp(m - sub), 0.0)
            l = corr * l + p.sum(axis=1)
            o = corr[:, None] * o + p @ vh[j0:j1]
            m = m_new
        ok = l > 0
        out[i0:i1][ok] = o[ok] / l[ok][:, None]
        lse[i0:i1][ok] = m[ok] + np.log(l[ok])
    return out, lse
