"""Fused exact-attention forward for AMD Instinct MI355X (gfx950).

Thin Python binding over the C ABI of ``libfa.so`` (include/fa.h).  torch is
used only to own device memory and to name the current stream; every step of
the computation runs in the library's HIP kernels.

    o, lse = attention(q, k, v, causal=True)                      # [B,N,H,d]
    o, lse = attention(q, k, v, causal=True, cu_seqlens_q=cu,     # packed
                       max_seqlen_q=n_max)
    o, lse = decode(q, k_cache, v_cache, cache_seqlens)           # split-KV
    o, lse = combine(o_part, lse_part)                            # LSE merge
"""
from __future__ import annotations

import math

import torch

from ._lib import FA_DTYPE_BF16, FA_DTYPE_F32, NOALLOC_SCRATCH_BYTES, FaError, check, load

__all__ = ["attention", "attention_fp8", "decode", "combine", "decode_workspace_size", "FaError", "load"]

_OUT_DTYPES = {torch.bfloat16: FA_DTYPE_BF16, torch.float32: FA_DTYPE_F32}


def _stream(stream):
    return torch.cuda.current_stream() if stream is None else stream


def _stream_handle(stream) -> int:
    return _stream(stream).cuda_stream


def _empty(shape, dtype, device, stream):
    """A new tensor owned by the stream the library's kernels run on, so that
    torch's caching allocator cannot hand its memory to work on another stream
    while those kernels still use it."""
    with torch.cuda.stream(_stream(stream)):
        return torch.empty(shape, dtype=dtype, device=device)


def _ptr(t):
    return None if t is None else t.data_ptr()


def _need(t, name, dtype, ndim=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions, got {t.dim()}")


def attention(q, k, v, *, causal: bool = False, scale: float | None = None,
              cu_seqlens_q=None, cu_seqlens_k=None, max_seqlen_q: int | None = None,
              max_seqlen_k: int | None = None, out=None, lse=None,
              out_dtype=torch.bfloat16, window=(-1, -1), softcap: float = 0.0,
              alibi_slopes=None, stream=None):
    """softmax(q k^T * scale) v and its row logsumexp.

    Fixed length: q [B, Nq, Hq, d], k/v [B, Nk, Hkv, d] -> o [B, Nq, Hq, d],
    lse [B, Nq, Hq].  Packed (cu_seqlens_q given, int32 [n+1]): q [Tq, Hq, d],
    k/v [Tk, Hkv, d] -> o [Tq, Hq, d], lse [Tq, Hq]; max_seqlen_q/k must bound
    the sequence lengths (read from the offsets on the host when omitted).

    Score variants (``fa_fwd_ext``): ``window`` = (left, right) admissible
    keys around the aligned diagonal (negative = open), ``softcap`` > 0 caps
    the scaled scores with tanh, ``alibi_slopes`` (fp32 [Hq] or [B, Hq]) adds
    -slope |i + Lk - Lq - j|.
    """
    lib = load()
    varlen = cu_seqlens_q is not None
    ndim = 3 if varlen else 4
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, n, torch.bfloat16, ndim)
    if out_dtype not in _OUT_DTYPES:
        raise TypeError("out_dtype must be torch.bfloat16 or torch.float32")
    if k.shape != v.shape:
        raise ValueError("k and v must have the same shape")
    d = q.shape[-1]
    if k.shape[-1] != d:
        raise ValueError("q and k head dims differ")
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    if varlen:
        _need(cu_seqlens_q, "cu_seqlens_q", torch.int32, 1)
        if cu_seqlens_k is not None:
            _need(cu_seqlens_k, "cu_seqlens_k", torch.int32, 1)
        batch = cu_seqlens_q.numel() - 1
        if max_seqlen_q is None:
            max_seqlen_q = int(torch.diff(cu_seqlens_q).max().item()) if batch > 0 else 0
        if max_seqlen_k is None:
            ck = cu_seqlens_q if cu_seqlens_k is None else cu_seqlens_k
            max_seqlen_k = int(torch.diff(ck).max().item()) if batch > 0 else 0
        hq, hkv = q.shape[1], k.shape[1]
        nq, nk = 0, 0
        lse_shape = (q.shape[0], hq)
    else:
        batch, nq, hq, _ = q.shape
        nk, hkv = k.shape[1], k.shape[2]
        if k.shape[0] != batch:
            raise ValueError("q and k batch sizes differ")
        max_seqlen_q = max_seqlen_k = 0
        lse_shape = (batch, nq, hq)
    if out is None:
        out = _empty(q.shape, out_dtype, q.device, stream)
    else:
        _need(out, "out", out_dtype, ndim)
        if out.shape != q.shape:
            raise ValueError("out must have q's shape")
    if lse is None:
        lse = _empty(lse_shape, torch.float32, q.device, stream)
    else:
        _need(lse, "lse", torch.float32)
        if tuple(lse.shape) != lse_shape:
            raise ValueError(f"lse must have shape {lse_shape}")
    left, right = (int(window[0]), int(window[1]))
    ext = left >= 0 or right >= 0 or softcap or alibi_slopes is not None
    if not ext:
        st = lib.fa_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), batch, hq, hkv, nq, nk,
                        d, scale, int(bool(causal)), _ptr(cu_seqlens_q), _ptr(cu_seqlens_k),
                        int(max_seqlen_q), int(max_seqlen_k), _OUT_DTYPES[out_dtype],
                        _stream_handle(stream))
        check(st, "fa_fwd")
        return out, lse
    astride = 0
    if alibi_slopes is not None:
        _need(alibi_slopes, "alibi_slopes", torch.float32)
        if tuple(alibi_slopes.shape) == (hq,):
            astride = 0
        elif tuple(alibi_slopes.shape) == (batch, hq):
            astride = hq
        else:
            raise ValueError("alibi_slopes must be [heads_q] or [batch, heads_q]")
    st = lib.fa_fwd_ext(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), batch, hq, hkv, nq, nk,
                        d, scale, int(bool(causal)), _ptr(cu_seqlens_q), _ptr(cu_seqlens_k),
                        int(max_seqlen_q), int(max_seqlen_k), left, right, float(softcap),
                        _ptr(alibi_slopes), astride, _OUT_DTYPES[out_dtype],
                        _stream_handle(stream))
    check(st, "fa_fwd_ext")
    return out, lse


def _fp8_codes(t, name, ndim):
    if isinstance(t, torch.Tensor) and t.dtype == torch.float8_e4m3fn:
        t = t.view(torch.uint8)
    _need(t, name, torch.uint8, ndim)
    return t


def attention_fp8(q, k, v, *, q_descale: float = 1.0, k_descale: float = 1.0,
                  v_descale: float = 1.0, causal: bool = False, scale: float | None = None,
                  cu_seqlens_q=None, cu_seqlens_k=None, max_seqlen_q: int | None = None,
                  max_seqlen_k: int | None = None, out=None, lse=None,
                  out_dtype=torch.bfloat16, stream=None):
    """``attention`` of FP8 inputs (``fa_fwd_fp8``): q, k, v hold E4M3 codes
    (torch.uint8 or torch.float8_e4m3fn, same shapes as ``attention``; head
    dim 128) and the real tensors are q_descale * q, k_descale * k and
    v_descale * v.  Returns (o, lse) of the real tensors."""
    lib = load()
    varlen = cu_seqlens_q is not None
    ndim = 3 if varlen else 4
    q, k, v = (_fp8_codes(t, n, ndim) for t, n in ((q, "q"), (k, "k"), (v, "v")))
    if out_dtype not in _OUT_DTYPES:
        raise TypeError("out_dtype must be torch.bfloat16 or torch.float32")
    if k.shape != v.shape:
        raise ValueError("k and v must have the same shape")
    d = q.shape[-1]
    if k.shape[-1] != d:
        raise ValueError("q and k head dims differ")
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    if varlen:
        _need(cu_seqlens_q, "cu_seqlens_q", torch.int32, 1)
        if cu_seqlens_k is not None:
            _need(cu_seqlens_k, "cu_seqlens_k", torch.int32, 1)
        batch = cu_seqlens_q.numel() - 1
        if max_seqlen_q is None:
            max_seqlen_q = int(torch.diff(cu_seqlens_q).max().item()) if batch > 0 else 0
        if max_seqlen_k is None:
            ck = cu_seqlens_q if cu_seqlens_k is None else cu_seqlens_k
            max_seqlen_k = int(torch.diff(ck).max().item()) if batch > 0 else 0
        hq, hkv, nq, nk = q.shape[1], k.shape[1], 0, 0
        lse_shape = (q.shape[0], hq)
    else:
        batch, nq, hq, _ = q.shape
        nk, hkv = k.shape[1], k.shape[2]
        if k.shape[0] != batch:
            raise ValueError("q and k batch sizes differ")
        max_seqlen_q = max_seqlen_k = 0
        lse_shape = (batch, nq, hq)
    if out is None:
        out = _empty(q.shape, out_dtype, q.device, stream)
    else:
        _need(out, "out", out_dtype, ndim)
        if out.shape != q.shape:
            raise ValueError("out must have q's shape")
    if lse is None:
        lse = _empty(lse_shape, torch.float32, q.device, stream)
    else:
        _need(lse, "lse", torch.float32)
        if tuple(lse.shape) != lse_shape:
            raise ValueError(f"lse must have shape {lse_shape}")
    st = lib.fa_fwd_fp8(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), batch, hq, hkv, nq, nk,
                        d, scale, float(q_descale), float(k_descale), float(v_descale),
                        int(bool(causal)), _ptr(cu_seqlens_q), _ptr(cu_seqlens_k),
                        int(max_seqlen_q), int(max_seqlen_k), _OUT_DTYPES[out_dtype],
                        _stream_handle(stream))
    check(st, "fa_fwd_fp8")
    return out, lse


def attention_backward(q, k, v, out, lse, dout, *, causal: bool = False,
                       scale: float | None = None, cu_seqlens_q=None, cu_seqlens_k=None,
                       max_seqlen_q: int | None = None, max_seqlen_k: int | None = None,
                       grad_dtype=torch.float32, workspace=None, stream=None):
    """Gradients (dq, dk, dv) of <dout, out> for ``attention``'s forward, given
    its output and logsumexp.  Shapes and conventions as ``attention``;
    dout has out's shape and dtype bf16.  ``workspace`` (uint8 device tensor)
    is allocated when omitted."""
    lib = load()
    varlen = cu_seqlens_q is not None
    ndim = 3 if varlen else 4
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (out, "out"), (dout, "dout")):
        _need(t, n, torch.bfloat16, ndim)
    _need(lse, "lse", torch.float32)
    if grad_dtype not in _OUT_DTYPES:
        raise TypeError("grad_dtype must be torch.bfloat16 or torch.float32")
    if k.shape != v.shape or out.shape != q.shape or dout.shape != q.shape:
        raise ValueError("k/v and q/out/dout shapes must match")
    d = q.shape[-1]
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    if varlen:
        _need(cu_seqlens_q, "cu_seqlens_q", torch.int32, 1)
        if cu_seqlens_k is not None:
            _need(cu_seqlens_k, "cu_seqlens_k", torch.int32, 1)
        batch = cu_seqlens_q.numel() - 1
        if max_seqlen_q is None:
            max_seqlen_q = int(torch.diff(cu_seqlens_q).max().item()) if batch > 0 else 0
        if max_seqlen_k is None:
            ck = cu_seqlens_q if cu_seqlens_k is None else cu_seqlens_k
            max_seqlen_k = int(torch.diff(ck).max().item()) if batch > 0 else 0
        hq, hkv = q.shape[1], k.shape[1]
        nq, nk = 0, 0
        rows_q = max_seqlen_q
        lse_shape = (q.shape[0], hq)
    else:
        batch, nq, hq, _ = q.shape
        nk, hkv = k.shape[1], k.shape[2]
        max_seqlen_q = max_seqlen_k = 0
        rows_q = nq
        lse_shape = (batch, nq, hq)
    if tuple(lse.shape) != lse_shape:
        raise ValueError(f"lse must have shape {lse_shape}")
    need = lib.fa_bwd_workspace_size(batch, hq, rows_q)
    if workspace is None:
        workspace = _empty(max(need, 16), torch.uint8, q.device, stream)
    else:
        _need(workspace, "workspace", torch.uint8)
    dq = _empty(q.shape, grad_dtype, q.device, stream)
    dk = _empty(k.shape, grad_dtype, q.device, stream)
    dv = _empty(v.shape, grad_dtype, q.device, stream)
    st = lib.fa_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(dout), _ptr(lse), _ptr(dq),
                    _ptr(dk), _ptr(dv), batch, hq, hkv, nq, nk, d, scale, int(bool(causal)),
                    _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), int(max_seqlen_q), int(max_seqlen_k),
                    _OUT_DTYPES[grad_dtype], _ptr(workspace), workspace.numel(),
                    _stream_handle(stream))
    check(st, "fa_bwd")
    return dq, dk, dv


def bwd_workspace_size(batch: int, heads_q: int, max_seqlen_q: int) -> int:
    return int(load().fa_bwd_workspace_size(batch, heads_q, max_seqlen_q))


def decode_workspace_size(batch: int, heads_q: int, max_cache_len: int, head_dim: int,
                          chunk: int = 0) -> int:
    return int(load().fa_decode_workspace_size(batch, heads_q, max_cache_len, head_dim, chunk))


def decode(q, k_cache, v_cache, cache_seqlens, *, scale: float | None = None, chunk: int = 0,
           out=None, lse=None, workspace=None, out_dtype=torch.bfloat16, stream=None):
    """One query per sequence against a KV cache, split over key chunks.

    q [B, Hq, d]; k_cache/v_cache [B, Ncache, Hkv, d]; cache_seqlens int32 [B]
    -> o [B, Hq, d], lse [B, Hq].  ``workspace`` (uint8 device tensor) is
    allocated when omitted.
    """
    lib = load()
    _need(q, "q", torch.bfloat16, 3)
    _need(k_cache, "k_cache", torch.bfloat16, 4)
    _need(v_cache, "v_cache", torch.bfloat16, 4)
    _need(cache_seqlens, "cache_seqlens", torch.int32, 1)
    if out_dtype not in _OUT_DTYPES:
        raise TypeError("out_dtype must be torch.bfloat16 or torch.float32")
    batch, hq, d = q.shape
    if k_cache.shape != v_cache.shape or k_cache.shape[0] != batch or k_cache.shape[3] != d:
        raise ValueError("cache shapes do not match q")
    if cache_seqlens.numel() != batch:
        raise ValueError("cache_seqlens must have one entry per sequence")
    ncache, hkv = k_cache.shape[1], k_cache.shape[2]
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    need = lib.fa_decode_workspace_size(batch, hq, ncache, d, chunk)
    if workspace is None:
        workspace = _empty(max(need, 16), torch.uint8, q.device, stream)
    else:
        _need(workspace, "workspace", torch.uint8)
    if out is None:
        out = _empty(q.shape, out_dtype, q.device, stream)
    else:
        _need(out, "out", out_dtype, 3)
        if out.shape != q.shape:
            raise ValueError("out must have q's shape")
    if lse is None:
        lse = _empty((batch, hq), torch.float32, q.device, stream)
    else:
        _need(lse, "lse", torch.float32, 2)
        if tuple(lse.shape) != (batch, hq):
            raise ValueError(f"lse must have shape {(batch, hq)}")
    st = lib.fa_fwd_decode_splitkv(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(cache_seqlens),
                                   _ptr(out), _ptr(lse), batch, hq, hkv, ncache, d, scale,
                                   int(chunk), _ptr(workspace), workspace.numel(),
                                   _OUT_DTYPES[out_dtype], _stream_handle(stream))
    check(st, "fa_fwd_decode_splitkv")
    return out, lse


def decode_kvcache_workspace_size(batch: int, heads_q: int, max_cache_len: int, head_dim: int,
                                  chunk: int = 0) -> int:
    return int(load().fa_decode_kvcache_workspace_size(batch, heads_q, max_cache_len, head_dim,
                                                       chunk))


def _kvcache_args(q, k_cache, v_cache, cache_seqlens, k_new, v_new, block_table, rotary_cos,
                  rotary_sin, out_dtype):
    """Checks of a KV-cache decode call; returns its sizes."""
    _need(q, "q", torch.bfloat16, 3)
    _need(k_cache, "k_cache", torch.bfloat16, 4)
    _need(v_cache, "v_cache", torch.bfloat16, 4)
    _need(cache_seqlens, "cache_seqlens", torch.int32, 1)
    if out_dtype not in _OUT_DTYPES:
        raise TypeError("out_dtype must be torch.bfloat16 or torch.float32")
    batch, hq, d = q.shape
    if k_cache.shape != v_cache.shape or k_cache.shape[3] != d:
        raise ValueError("cache shapes do not match q")
    if cache_seqlens.numel() != batch:
        raise ValueError("cache_seqlens must have one entry per sequence")
    hkv = k_cache.shape[2]
    if (k_new is None) != (v_new is None):
        raise ValueError("k_new and v_new go together")
    if k_new is not None:
        for t, n in ((k_new, "k_new"), (v_new, "v_new")):
            _need(t, n, torch.bfloat16, 3)
            if tuple(t.shape) != (batch, hkv, d):
                raise ValueError(f"{n} must be [batch, heads_kv, head_dim]")
    if block_table is not None:
        _need(block_table, "block_table", torch.int32, 2)
        if block_table.shape[0] != batch:
            raise ValueError("block_table must have one row per sequence")
        num_blocks, page = k_cache.shape[0], k_cache.shape[1]
        max_blocks = block_table.shape[1]
        cap = max_blocks * page
    else:
        if k_cache.shape[0] != batch:
            raise ValueError("contiguous caches have one slice per sequence")
        num_blocks = page = max_blocks = 0
        cap = k_cache.shape[1]
    if (rotary_cos is None) != (rotary_sin is None):
        raise ValueError("rotary_cos and rotary_sin go together")
    rdim = max_pos = 0
    if rotary_cos is not None:
        _need(rotary_cos, "rotary_cos", torch.float32, 2)
        _need(rotary_sin, "rotary_sin", torch.float32, 2)
        if rotary_cos.shape != rotary_sin.shape:
            raise ValueError("rotary tables differ in shape")
        max_pos, rdim = rotary_cos.shape[0], 2 * rotary_cos.shape[1]
    return batch, hq, hkv, d, cap, max_blocks, page, num_blocks, rdim, max_pos


def _check_out_lse(out, lse, q, out_dtype):
    batch, hq = q.shape[0], q.shape[1]
    _need(out, "out", out_dtype, 3)
    if out.shape != q.shape:
        raise ValueError("out must have q's shape")
    _need(lse, "lse", torch.float32, 2)
    if tuple(lse.shape) != (batch, hq):
        raise ValueError(f"lse must have shape {(batch, hq)}")


def decode_kvcache(q, k_cache, v_cache, cache_seqlens, *, k_new=None, v_new=None,
                   block_table=None, rotary_cos=None, rotary_sin=None,
                   rotary_interleaved: bool = False, scale: float | None = None, chunk: int = 0,
                   out=None, lse=None, workspace=None, out_dtype=torch.bfloat16, stream=None):
    """One decode step that updates the cache in place (``fa_fwd_decode_kvcache``).

    q [B, Hq, d]; k_new/v_new [B, Hkv, d] or None; cache_seqlens int32 [B]
    (tokens cached before the call; not modified).  Contiguous caches are
    [B, Ncache, Hkv, d]; with ``block_table`` (int32 [B, max_blocks]) they are
    paged [num_blocks, page_size, Hkv, d].  ``rotary_cos``/``rotary_sin`` are
    fp32 [max_pos, rotary_dim / 2].  Returns (o [B, Hq, d], lse [B, Hq]).
    """
    lib = load()
    batch, hq, hkv, d, cap, max_blocks, page, num_blocks, rdim, max_pos = _kvcache_args(
        q, k_cache, v_cache, cache_seqlens, k_new, v_new, block_table, rotary_cos, rotary_sin,
        out_dtype)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    need = lib.fa_decode_kvcache_workspace_size(batch, hq, cap, d, chunk)
    if workspace is None:
        workspace = _empty(max(need, 16), torch.uint8, q.device, stream)
    else:
        _need(workspace, "workspace", torch.uint8)
    if out is None:
        out = _empty(q.shape, out_dtype, q.device, stream)
    if lse is None:
        lse = _empty((batch, hq), torch.float32, q.device, stream)
    _check_out_lse(out, lse, q, out_dtype)
    st = lib.fa_fwd_decode_kvcache(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_new), _ptr(v_new), _ptr(cache_seqlens),
        _ptr(block_table), max_blocks, page, num_blocks, _ptr(rotary_cos), _ptr(rotary_sin), rdim,
        max_pos, int(bool(rotary_interleaved)), _ptr(out), _ptr(lse), batch, hq, hkv, cap, d,
        scale, int(chunk), _ptr(workspace), workspace.numel(), _OUT_DTYPES[out_dtype],
        _stream_handle(stream))
    check(st, "fa_fwd_decode_kvcache")
    return out, lse


def decode_kvcache_noalloc(q, k_cache, v_cache, cache_seqlens, out, lse, *, k_new=None,
                           v_new=None, block_table=None, rotary_cos=None, rotary_sin=None,
                           rotary_interleaved: bool = False, scale: float | None = None,
                           chunk: int = 0, stream=None):
    """``decode_kvcache`` without any allocation (``fa_fwd_decode_kvcache_noalloc``):
    the caller passes ``out`` [B, Hq, d] (bf16 or fp32, which sets the output
    dtype) and ``lse`` fp32 [B, Hq]; the partials live in the library's own
    per-device scratch of ``NOALLOC_SCRATCH_BYTES``.  Calls that can overlap on
    one device race on that scratch."""
    lib = load()
    if out is None or lse is None:
        raise ValueError("decode_kvcache_noalloc writes into caller-provided out and lse")
    out_dtype = out.dtype
    batch, hq, hkv, d, cap, max_blocks, page, num_blocks, rdim, max_pos = _kvcache_args(
        q, k_cache, v_cache, cache_seqlens, k_new, v_new, block_table, rotary_cos, rotary_sin,
        out_dtype)
    _check_out_lse(out, lse, q, out_dtype)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    st = lib.fa_fwd_decode_kvcache_noalloc(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_new), _ptr(v_new), _ptr(cache_seqlens),
        _ptr(block_table), max_blocks, page, num_blocks, _ptr(rotary_cos), _ptr(rotary_sin), rdim,
        max_pos, int(bool(rotary_interleaved)), _ptr(out), _ptr(lse), batch, hq, hkv, cap, d,
        scale, int(chunk), _OUT_DTYPES[out_dtype], _stream_handle(stream))
    check(st, "fa_fwd_decode_kvcache_noalloc")
    return out, lse


def combine(o_part, lse_part, *, out=None, lse=None, out_dtype=torch.float32, stream=None):
    """LSE-weighted merge: o_part [rows, S, d] fp32, lse_part [rows, S] fp32
    (-inf = empty split) -> o [rows, d], lse [rows]."""
    lib = load()
    _need(o_part, "o_part", torch.float32, 3)
    _need(lse_part, "lse_part", torch.float32, 2)
    rows, n_splits, d = o_part.shape
    if tuple(lse_part.shape) != (rows, n_splits):
        raise ValueError("lse_part must be [rows, n_splits]")
    if out_dtype not in _OUT_DTYPES:
        raise TypeError("out_dtype must be torch.bfloat16 or torch.float32")
    if out is None:
        out = _empty((rows, d), out_dtype, o_part.device, stream)
    else:
        _need(out, "out", out_dtype, 2)
        if tuple(out.shape) != (rows, d):
            raise ValueError(f"out must have shape {(rows, d)}")
    if lse is None:
        lse = _empty((rows,), torch.float32, o_part.device, stream)
    else:
        _need(lse, "lse", torch.float32, 1)
        if tuple(lse.shape) != (rows,):
            raise ValueError(f"lse must have shape {(rows,)}")
    st = lib.fa_combine(_ptr(o_part), _ptr(lse_part), rows, n_splits, d, _ptr(out), _ptr(lse),
                        _OUT_DTYPES[out_dtype], _stream_handle(stream))
    check(st, "fa_combine")
    return out, lse
