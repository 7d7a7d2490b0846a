"""Seeded synthetic inputs for the attention-forward workloads.

This module only draws numbers and shapes: it holds none of the attention
arithmetic, so that both the fp64 CPU oracle (``oracle/``) and the HIP path
(``exact_attention_84_amd``) can be fed identical input bytes from it without
sharing any code with each other.

Every tensor is drawn as float32 N(0, 1) from
``numpy.random.default_rng(SeedSequence([seed, workload_id, tensor_id, slice]))``
and rounded to bfloat16 with round-to-nearest-even.  Tensors are returned as
``uint16`` arrays holding the bfloat16 bit patterns, so that no side performs
a second rounding.

Workloads (shapes follow the long-sequence, GQA, varlen and KV-cache decode
regimes discussed on the pages "FlashAttention — IO 感知的精确注意力 kernel",
§1 capability table and §1 usage snippet, and "推理优化 | FlashAttention 1-4 详解",
§原算法 (the 8K-sequence motivation)):

  1  single head      B=1, H=1, N=256, d=64, non-causal
  2  batched MHA      B=4, H=16, N=2048, d=128, non-causal and causal
  3  long causal GQA  B=1, Hq=32, Hkv=8, N=8192, d=128, K drawn then scaled by 2
  4  varlen causal    16 sequences, lengths uniform on [128, 4096], Hq=32, Hkv=8
  5  split-KV decode  B=64, Hq=32, Hkv=8, one query per sequence, cache lengths
                      uniform on [16384, 32768], cache allocated to 32768
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

# Tensor ids inside a workload's seed sequence.
T_Q, T_K, T_V, T_LEN, T_DO = 0, 1, 2, 3, 4


@dataclasses.dataclass(frozen=True)
class Workload:
    wid: int
    name: str
    batch: int
    heads_q: int
    heads_kv: int
    seqlen_q: int          # fixed mode; 1 for decode; max length for varlen
    seqlen_k: int          # fixed mode; cache allocation for decode
    head_dim: int
    causal: bool
    kind: str              # "fixed" | "varlen" | "decode"
    k_mult: float = 1.0
    len_lo: int = 0        # varlen / decode length range (inclusive)
    len_hi: int = 0

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)


WORKLOADS = {
    1: Workload(1, "single_head_n256_d64", 1, 1, 1, 256, 256, 64, False, "fixed"),
    2: Workload(2, "mha_b4_h16_n2048_d128", 4, 16, 16, 2048, 2048, 128, False, "fixed"),
    3: Workload(3, "gqa_causal_b1_h32kv8_n8192_d128", 1, 32, 8, 8192, 8192, 128, True,
                "fixed", k_mult=2.0),
    4: Workload(4, "varlen_causal_16seq_h32kv8_d128", 16, 32, 8, 4096, 4096, 128, True,
                "varlen", len_lo=128, len_hi=4096),
    5: Workload(5, "decode_b64_h32kv8_cache32k_d128", 64, 32, 8, 1, 32768, 128, False,
                "decode", len_lo=16384, len_hi=32768),
}


def _rng(seed: int, wid: int, tensor: int, slc: int = 0) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([seed, wid, tensor, slc]))


def round_f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round finite float32 values to bfloat16 (nearest, ties to even); return
    uint16 bits.  (Only NaN payloads could wrap in the 32-bit add.)"""
    x = np.ascontiguousarray(x, dtype=np.float32)
    b = x.view(np.uint32).copy()
    b += np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1))
    return (b >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def normal_bf16(seed: int, wid: int, tensor: int, shape, slc: int = 0,
                mult: float = 1.0) -> np.ndarray:
    """float32 N(0,1) draw (times ``mult``) rounded to bfloat16 bits."""
    x = _rng(seed, wid, tensor, slc).standard_normal(size=shape, dtype=np.float32)
    if mult != 1.0:
        x *= np.float32(mult)
    return round_f32_to_bf16_bits(x)


def uniform_lengths(seed: int, wid: int, n: int, lo: int, hi: int) -> np.ndarray:
    """n integers uniform on the inclusive range [lo, hi] (int32)."""
    return _rng(seed, wid, T_LEN).integers(lo, hi + 1, size=n).astype(np.int32)


def prefix_sums(lengths: np.ndarray) -> np.ndarray:
    """int32 [n+1] exclusive prefix sums (cu_seqlens)."""
    cu = np.zeros(len(lengths) + 1, dtype=np.int64)
    cu[1:] = np.cumsum(lengths)
    return cu.astype(np.int32)


def make_fixed(batch, heads_q, heads_kv, seqlen_q, seqlen_k, head_dim, *, seed=0,
               wid=0, k_mult=1.0):
    """q [B,Nq,Hq,d], k/v [B,Nk,Hkv,d] as bf16 bits; one slice per batch entry."""
    q = np.empty((batch, seqlen_q, heads_q, head_dim), np.uint16)
    k = np.empty((batch, seqlen_k, heads_kv, head_dim), np.uint16)
    v = np.empty((batch, seqlen_k, heads_kv, head_dim), np.uint16)
    for b in range(batch):
        q[b] = normal_bf16(seed, wid, T_Q, q.shape[1:], b)
        k[b] = normal_bf16(seed, wid, T_K, k.shape[1:], b, k_mult)
        v[b] = normal_bf16(seed, wid, T_V, v.shape[1:], b)
    return q, k, v


def make_varlen(lengths_q, lengths_k, heads_q, heads_kv, head_dim, *, seed=0, wid=0,
                k_mult=1.0):
    """Packed q [sum Lq, Hq, d], k/v [sum Lk, Hkv, d] plus int32 cu_seqlens."""
    lengths_q = np.asarray(lengths_q, np.int32)
    lengths_k = np.asarray(lengths_k, np.int32)
    cu_q, cu_k = prefix_sums(lengths_q), prefix_sums(lengths_k)
    q = np.empty((int(cu_q[-1]), heads_q, head_dim), np.uint16)
    k = np.empty((int(cu_k[-1]), heads_kv, head_dim), np.uint16)
    v = np.empty((int(cu_k[-1]), heads_kv, head_dim), np.uint16)
    for s in range(len(lengths_q)):
        q[cu_q[s]:cu_q[s + 1]] = normal_bf16(seed, wid, T_Q, (lengths_q[s], heads_q, head_dim), s)
        k[cu_k[s]:cu_k[s + 1]] = normal_bf16(seed, wid, T_K, (lengths_k[s], heads_kv, head_dim),
                                             s, k_mult)
        v[cu_k[s]:cu_k[s + 1]] = normal_bf16(seed, wid, T_V, (lengths_k[s], heads_kv, head_dim), s)
    return q, k, v, cu_q, cu_k


def make_dout(q_shape, *, seed=0, wid=0, cu_q=None) -> np.ndarray:
    """Upstream gradient dO with the query tensor's shape (bf16 bits): one
    slice per batch entry, or per packed sequence when ``cu_q`` is given."""
    do = np.empty(q_shape, np.uint16)
    if cu_q is None:
        for b in range(q_shape[0]):
            do[b] = normal_bf16(seed, wid, T_DO, q_shape[1:], b)
    else:
        for s in range(len(cu_q) - 1):
            a, e = int(cu_q[s]), int(cu_q[s + 1])
            do[a:e] = normal_bf16(seed, wid, T_DO, (e - a,) + tuple(q_shape[1:]), s)
    return do


# FP8 inputs: N(0,1) draws times a per-tensor multiplier, cast to E4M3 codes by
# torch's float8_e4m3fn conversion (nearest, ties to even), with descale =
def make_rising(batch, heads_q, heads_kv, seqlen, head_dim, *, seed=0, wid=0,
                lift=4.0, slope=1.0 / 16):
    """make_fixed's bf16 tensors with a ramp built in: component 0 of every
    query is ``lift`` and component 0 of key j is ``slope * j``, so every
    row's scores grow along the keys on top of the N(0,1) terms."""
    q, k, v = make_fixed(batch, heads_q, heads_kv, seqlen, seqlen, head_dim, seed=seed, wid=wid)
    q[..., 0] = round_f32_to_bf16_bits(np.float32([lift]))[0]
    ramp = round_f32_to_bf16_bits(np.float32(slope) * np.arange(seqlen, dtype=np.float32))
    k[..., 0] = ramp[None, :, None]
    return q, k, v


# 1 / multiplier so that descale * decoded codes is N(0,1)-shaped (times
# k_mult for K).  The multipliers put the bulk of each tensor in E4M3's normal
# range; draws are clipped to +-440 first (E4M3's largest finite value is 448).
FP8_MULT = {T_Q: 32.0, T_K: 16.0, T_V: 64.0}


def normal_fp8(seed: int, wid: int, tensor: int, shape, slc: int = 0,
               mult: float = 1.0) -> np.ndarray:
    """uint8 E4M3 codes of a N(0,1) draw times ``mult`` times the tensor's
    FP8 multiplier."""
    import torch
    x = _rng(seed, wid, tensor, slc).standard_normal(size=shape, dtype=np.float32)
    x *= np.float32(mult * FP8_MULT[tensor])
    np.clip(x, -440.0, 440.0, out=x)
    return torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def make_fixed_fp8(batch, heads_q, heads_kv, seqlen_q, seqlen_k, head_dim, *, seed=0,
                   wid=0, k_mult=1.0):
    """q8 [B,Nq,Hq,d], k8/v8 [B,Nk,Hkv,d] as E4M3 codes plus the three
    per-tensor descales (q, k, v); one slice per batch entry."""
    q = np.empty((batch, seqlen_q, heads_q, head_dim), np.uint8)
    k = np.empty((batch, seqlen_k, heads_kv, head_dim), np.uint8)
    v = np.empty((batch, seqlen_k, heads_kv, head_dim), np.uint8)
    for b in range(batch):
        q[b] = normal_fp8(seed, wid, T_Q, q.shape[1:], b)
        k[b] = normal_fp8(seed, wid, T_K, k.shape[1:], b, k_mult)
        v[b] = normal_fp8(seed, wid, T_V, v.shape[1:], b)
    descales = tuple(1.0 / FP8_MULT[t] for t in (T_Q, T_K, T_V))
    return q, k, v, descales


def make_rising_fp8(batch, heads_q, heads_kv, seqlen, head_dim, *, seed=0, wid=0,
                    lift=8.0, top=28.0):
    """make_fixed_fp8's E4M3 codes with a ramp built in: component 0 of every
    query is ``lift`` and component 0 of key j is ``top * j / seqlen`` (real
    values, before the per-tensor multipliers), so every row's scores grow
    along the keys.  Returns (q8, k8, v8, descales)."""
    import torch
    q, k, v, ds = make_fixed_fp8(batch, heads_q, heads_kv, seqlen, seqlen, head_dim, seed=seed,
                                 wid=wid)

    def code(x):
        x = np.clip(np.asarray(x, np.float32), -440.0, 440.0)
        return torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()

    q[..., 0] = code([lift * FP8_MULT[T_Q]])[0]
    ramp = np.float32(top / seqlen) * np.arange(seqlen, dtype=np.float32)
    k[..., 0] = code(ramp * np.float32(FP8_MULT[T_K]))[None, :, None]
    return q, k, v, ds


def make_varlen_fp8(lengths_q, lengths_k, heads_q, heads_kv, head_dim, *, seed=0, wid=0):
    """Packed E4M3 codes q8 [sum Lq, Hq, d], k8/v8 [sum Lk, Hkv, d], int32
    cu_seqlens and the per-tensor descales (q, k, v)."""
    lengths_q = np.asarray(lengths_q, np.int32)
    lengths_k = np.asarray(lengths_k, np.int32)
    cu_q, cu_k = prefix_sums(lengths_q), prefix_sums(lengths_k)
    q = np.empty((int(cu_q[-1]), heads_q, head_dim), np.uint8)
    k = np.empty((int(cu_k[-1]), heads_kv, head_dim), np.uint8)
    v = np.empty((int(cu_k[-1]), heads_kv, head_dim), np.uint8)
    for s in range(len(lengths_q)):
        q[cu_q[s]:cu_q[s + 1]] = normal_fp8(seed, wid, T_Q, (lengths_q[s], heads_q, head_dim), s)
        k[cu_k[s]:cu_k[s + 1]] = normal_fp8(seed, wid, T_K, (lengths_k[s], heads_kv, head_dim), s)
        v[cu_k[s]:cu_k[s + 1]] = normal_fp8(seed, wid, T_V, (lengths_k[s], heads_kv, head_dim), s)
    descales = tuple(1.0 / FP8_MULT[t] for t in (T_Q, T_K, T_V))
    return q, k, v, cu_q, cu_k, descales


BF16_NAN = np.uint16(0x7FC0)


def decode_q(batch, heads_q, head_dim, *, seed=0, wid=0) -> np.ndarray:
    """Decode queries q [B, Hq, d] (bf16 bits)."""
    q = np.empty((batch, heads_q, head_dim), np.uint16)
    for b in range(batch):
        q[b] = normal_bf16(seed, wid, T_Q, (heads_q, head_dim), b)
    return q


def decode_kv_slice(b, n, heads_kv, head_dim, *, seed=0, wid=0):
    """The n valid cache rows of sequence b: (k, v), each [n, Hkv, d] bf16 bits."""
    return (normal_bf16(seed, wid, T_K, (n, heads_kv, head_dim), b),
            normal_bf16(seed, wid, T_V, (n, heads_kv, head_dim), b))


def make_decode(batch, heads_q, heads_kv, cache_len, head_dim, cache_seqlens, *, seed=0,
                wid=0, tail="zero", workers=8):
    """q [B,Hq,d]; k/v caches [B,cache_len,Hkv,d]; rows past cache_seqlens[b] are
    zero (tail="zero") or NaN (tail="nan", to show they are never used)."""
    import concurrent.futures as cf
    cache_seqlens = np.asarray(cache_seqlens, np.int32)
    q = decode_q(batch, heads_q, head_dim, seed=seed, wid=wid)
    k = np.empty((batch, cache_len, heads_kv, head_dim), np.uint16)
    v = np.empty((batch, cache_len, heads_kv, head_dim), np.uint16)
    fill = BF16_NAN if tail == "nan" else np.uint16(0)

    def one(b):
        n = int(cache_seqlens[b])
        k[b, :n], v[b, :n] = decode_kv_slice(b, n, heads_kv, head_dim, seed=seed, wid=wid)
        k[b, n:] = fill
        v[b, n:] = fill

    with cf.ThreadPoolExecutor(max_workers=max(1, workers)) as ex:
        list(ex.map(one, range(batch)))
    return q, k, v


def workload_lengths(w: Workload, seed: int = 0) -> np.ndarray:
    """Per-sequence lengths of a varlen or decode workload."""
    return uniform_lengths(seed, w.wid, w.batch, w.len_lo, w.len_hi)


def make_workload(w: Workload, seed: int = 0, tail: str = "zero") -> dict:
    """All inputs of one workload as numpy arrays (bf16 bits, int32 metadata)."""
    if w.kind == "fixed":
        q, k, v = make_fixed(w.batch, w.heads_q, w.heads_kv, w.seqlen_q, w.seqlen_k,
                             w.head_dim, seed=seed, wid=w.wid, k_mult=w.k_mult)
        return dict(q=q, k=k, v=v)
    if w.kind == "varlen":
        lens = workload_lengths(w, seed)
        q, k, v, cu_q, cu_k = make_varlen(lens, lens, w.heads_q, w.heads_kv, w.head_dim,
                                          seed=seed, wid=w.wid, k_mult=w.k_mult)
        return dict(q=q, k=k, v=v, cu_q=cu_q, cu_k=cu_k, lengths=lens)
    lens = workload_lengths(w, seed)
    q, k, v = make_decode(w.batch, w.heads_q, w.heads_kv, w.seqlen_k, w.head_dim, lens,
                          seed=seed, wid=w.wid, tail=tail)
    return dict(q=q, k=k, v=v, cache_seqlens=lens)


def flops(w: Workload, lengths=None, causal=None) -> float:
    """Algorithmic forward flops: 4*Hq*Lq*Lk*d per sequence, halved when causal
    (the metric's convention), summed over sequences."""
    causal = w.causal if causal is None else causal
    f = 0.5 if causal else 1.0
    if w.kind == "fixed":
        return f * 4.0 * w.batch * w.heads_q * w.seqlen_q * w.seqlen_k * w.head_dim
    lengths = workload_lengths(w) if lengths is None else lengths
    if w.kind == "varlen":
        return float(sum(f * 4.0 * w.heads_q * int(n) * int(n) * w.head_dim for n in lengths))
    return float(sum(4.0 * w.heads_q * int(n) * w.head_dim for n in lengths))


def decode_bytes(w: Workload, lengths=None) -> float:
    """Algorithmic HBM bytes of a decode step: every valid K and V row once, plus
    q, O (bf16) and LSE (fp32)."""
    lengths = workload_lengths(w) if lengths is None else lengths
    kv = 2.0 * float(np.sum(lengths)) * w.heads_kv * w.head_dim * 2
    qo = 2.0 * w.batch * w.heads_q * w.head_dim * 2 + w.batch * w.heads_q * 4
    return kv + qo
