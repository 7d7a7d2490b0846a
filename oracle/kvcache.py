"""fp64 CPU oracle for one KV-cache decode step: rotary position embedding of
the new token's query and key, in-place append of its key and value to the
cache, and single-query attention over a contiguous or paged cache.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module.  The HIP
library never routes through it and shares no code with it.

The pages name these features and nothing more ("FlashAttention — IO 感知的精确
注意力 kernel", §1: the capability table lists in-place KV-cache append, paged
KV and split-KV decode, and the usage snippet's KV-cache call updates the cache
in place and applies rotary in the same call).  The readings taken:

  * Rotary position embedding rotates a vector x at position t pair by pair:
    the first r = rotary_dim components form r/2 pairs, and pair i turns by
    the angle whose cosine and sine the caller gives as cos[t, i], sin[t, i]:
        (a, b) -> (a cos - b sin,  b cos + a sin).
    Pairs are (x[i], x[i + r/2]) by default ("rotate half") or (x[2i],
    x[2i + 1]) when interleaved.  Components from r on are unchanged.
  * The cache of sequence b holds t_b = cache_seqlens[b] tokens before the
    call.  The new token sits at position t_b: its query and key are rotated
    at t_b, its key and value are written to cache row t_b, and attention
    covers rows [0, t_b + 1).  With no new key/value nothing is written and
    attention covers rows [0, t_b); rotary then still applies to the query.
  * Rotated query and key are rounded to bfloat16 (round to nearest even),
    the cache's storage type, before they are used.
  * Paged cache: row j of sequence b lives in physical block
    block_table[b][j // page_size], at row j % page_size of that block.
  * Attention itself is the single-query definition of ``oracle.exact``
    (every cached key admissible, grouped heads h -> h // (Hq / Hkv)).
"""
from __future__ import annotations

import numpy as np

from .exact import _group, head_attention, kv_head, to_f64


def to_bf16_rne(x) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 (8 significant bits),
    ties to even, returned as float64.  Finite normal inputs only."""
    x = np.asarray(x, np.float64)
    m, e = np.frexp(x)                    # x = m 2^e, 0.5 <= |m| < 1
    return np.ldexp(np.round(m * 256.0), e - 8)   # np.round: half to even


def bf16_bits(x) -> np.ndarray:
    """bfloat16-representable float64 values -> their uint16 bit patterns."""
    return (np.asarray(x, np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def rotary(x, cos_t, sin_t, rotary_dim: int, interleaved: bool = False) -> np.ndarray:
    """Rotate the last axis of x (float64) by the per-pair angles cos_t/sin_t
    [..., rotary_dim/2] (broadcast against x's leading axes)."""
    x = np.array(x, np.float64, copy=True)
    r = rotary_dim
    if r == 0:
        return x
    if interleaved:
        a, b = x[..., 0:r:2].copy(), x[..., 1:r:2].copy()
    else:
        a, b = x[..., : r // 2].copy(), x[..., r // 2: r].copy()
    ra = a * cos_t - b * sin_t
    rb = b * cos_t + a * sin_t
    if interleaved:
        x[..., 0:r:2], x[..., 1:r:2] = ra, rb
    else:
        x[..., : r // 2], x[..., r // 2: r] = ra, rb
    return x


def cache_row_index(b: int, j: int, block_table, page_size: int):
    """(first index, second index) of logical row j of sequence b: (b, j) in a
    contiguous cache [B, N, Hkv, d], (block, row) in a paged one
    [blocks, page_size, Hkv, d]."""
    if block_table is None:
        return b, j
    return int(block_table[b][j // page_size]), j % page_size


def gather_rows(cache, b: int, n: int, block_table, page_size: int) -> np.ndarray:
    """Logical rows [0, n) of sequence b as float64 [n, Hkv, d]."""
    if n == 0:
        return np.zeros((0,) + tuple(cache.shape[2:]))
    if block_table is None:
        return to_f64(cache[b, :n])
    j = np.arange(n)
    idx = [cache_row_index(b, int(x), block_table, page_size) for x in j[::page_size]]
    blocks = np.repeat([i[0] for i in idx], page_size)[:n]
    return to_f64(cache[blocks, j % page_size])


def kvcache_step(q, k_cache, v_cache, cache_seqlens, scale: float, k_new=None, v_new=None,
                 block_table=None, page_size: int = 0, rotary_cos=None, rotary_sin=None,
                 rotary_dim: int = 0, interleaved: bool = False):
    """One decode step.  q [B, Hq, d] and k_new/v_new [B, Hkv, d] as bf16 bits;
    caches as bf16 bits, contiguous [B, N, Hkv, d] or paged
    [blocks, page_size, Hkv, d] with block_table [B, max_blocks];
    rotary tables [max_pos, rotary_dim/2] (None: no rotary).

    Returns (O [B, Hq, d], LSE [B, Hq], k_cache', v_cache'), the caches as
    updated copies (bf16 bits).
    """
    qf = to_f64(q)
    bsz, hq, d = qf.shape
    hkv = k_cache.shape[2]
    g = _group(hq, hkv)
    k_out = np.array(k_cache, copy=True)
    v_out = np.array(v_cache, copy=True)
    use_rot = rotary_cos is not None and rotary_dim > 0
    out = np.zeros((bsz, hq, d))
    lse = np.full((bsz, hq), -np.inf)
    for b in range(bsz):
        t = int(cache_seqlens[b])
        qb = qf[b]
        if use_rot:
            cs, sn = np.asarray(rotary_cos, np.float64)[t], np.asarray(rotary_sin, np.float64)[t]
            qb = to_bf16_rne(rotary(qb, cs, sn, rotary_dim, interleaved))
        n = t
        if k_new is not None:
            kb = to_f64(k_new[b])
            if use_rot:
                kb = to_bf16_rne(rotary(kb, cs, sn, rotary_dim, interleaved))
            idx = cache_row_index(b, t, block_table, page_size)
            k_out[idx] = bf16_bits(kb)
            v_out[idx] = np.asarray(v_new[b])
            n = t + 1
        ks = gather_rows(k_out, b, n, block_table, page_size)
        vs = gather_rows(v_out, b, n, block_table, page_size)
        for h in range(hq):
            kh = kv_head(h, g)
            o, l = head_attention(qb[h][None, :], ks[:, kh], vs[:, kh], scale, causal=False)
            out[b, h] = o[0]
            lse[b, h] = l[0]
    return out, lse, k_out, v_out
