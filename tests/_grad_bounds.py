"""Error bounds of the backward's arithmetic, and the comparison against the
fp64 gradient oracle used by the GPU backward tests.

Bound, per element, derived from the arithmetic of the kernels (fp32
accumulation of bf16 MFMA products; P and dS rounded to bf16 before the
products that consume them; D = rowsum(dO * O) taken from the bf16 O that was
passed in):

  P relative error   eP  = |expm1(LSE_exact - LSE_in)|          (LSE input)
  dS error           eS  = (2^-8 + eP) |dS| + P |D_in - D_exact|
                           + P 2^-24 d sum_d |dO O|              (D in fp32)
  dQ                 scale (eS |K|)  + n_k 2^-24 scale (|dS| |K|)
  dK                 scale (eSᵀ |Q|) + n_q 2^-24 scale (|dS|ᵀ |Q|)
  dV                 (2^-8 + eP) Pᵀ |dO| + n_q 2^-24 Pᵀ |dO|

(products of absolute values are the worst case of each sum; grouped heads
add their bounds).  The test allows twice the bound plus 1e-6 of the
tensor's largest value, and for bf16 gradients half a bf16 ulp of the
exact value on top.  No NaN or Inf anywhere.
"""
import numpy as np

import oracle
import workloads as W
from _gpu_helpers import bf16_half_ulp

U_BF16 = 2.0 ** -8   # unit roundoff of bfloat16 (8-bit significand)
U_F32 = 2.0 ** -24


def bf16_bits_of(x):
    return W.round_f32_to_bf16_bits(np.asarray(x, np.float32))


def head_bounds(qh, kh, vh, doh, o_in, lse_in, scale, causal):
    """Error bounds (dQ [lq,d], dK [lk,d], dV [lk,d]) of one (sequence, head)."""
    lq, lk, d = qh.shape[0], kh.shape[0], qh.shape[1]
    p = oracle.probabilities(qh, kh, scale, causal)
    ds = oracle.softmax_backward(p, oracle.prob_grad(doh, vh))
    o_ex, lse_ex = oracle.head_attention(qh, kh, vh, scale, causal)
    fin = np.isfinite(lse_ex)
    e_p = np.zeros(lq)
    e_p[fin] = np.abs(np.expm1(lse_ex[fin] - lse_in[fin]))
    d_err = np.abs((doh * (o_in - o_ex)).sum(axis=1))
    d_acc = U_F32 * d * np.abs(doh * o_in).sum(axis=1)
    e_s = (U_BF16 + e_p)[:, None] * np.abs(ds) + p * (d_err + d_acc)[:, None]
    aq, ak, ado = np.abs(qh), np.abs(kh), np.abs(doh)
    bq = scale * (e_s @ ak) + lk * U_F32 * scale * (np.abs(ds) @ ak)
    bk = scale * (e_s.T @ aq) + lq * U_F32 * scale * (np.abs(ds).T @ aq)
    pd = p.T @ ado
    bv = (U_BF16 + e_p.max(initial=0.0)) * pd + lq * U_F32 * pd
    return bq, bk, bv


def fixed_bounds(q, k, v, do, o_in, lse_in, scale, causal):
    q, k, v, do = (W.bf16_bits_to_f32(x).astype(np.float64) for x in (q, k, v, do))
    bq, bk, bv = np.zeros(q.shape), np.zeros(k.shape), np.zeros(v.shape)
    g = q.shape[2] // k.shape[2]
    for b in range(q.shape[0]):
        for h in range(q.shape[2]):
            x = head_bounds(q[b, :, h], k[b, :, h // g], v[b, :, h // g], do[b, :, h],
                            o_in[b, :, h], lse_in[b, :, h], scale, causal)
            bq[b, :, h] = x[0]
            bk[b, :, h // g] += x[1]
            bv[b, :, h // g] += x[2]
    return bq, bk, bv


def varlen_bounds(q, k, v, do, o_in, lse_in, cu_q, cu_k, scale, causal):
    q, k, v, do = (W.bf16_bits_to_f32(x).astype(np.float64) for x in (q, k, v, do))
    bq, bk, bv = np.zeros(q.shape), np.zeros(k.shape), np.zeros(v.shape)
    g = q.shape[1] // k.shape[1]
    for s in range(len(cu_q) - 1):
        qa, qb, ka, kb = cu_q[s], cu_q[s + 1], cu_k[s], cu_k[s + 1]
        for h in range(q.shape[1]):
            x = head_bounds(q[qa:qb, h], k[ka:kb, h // g], v[ka:kb, h // g], do[qa:qb, h],
                            o_in[qa:qb, h], lse_in[qa:qb, h], scale, causal)
            bq[qa:qb, h] = x[0]
            bk[ka:kb, h // g] += x[1]
            bv[ka:kb, h // g] += x[2]
    return bq, bk, bv


def check_grad(name, got, ref, bound, bf16_out, what):
    got = np.asarray(got, np.float64)
    assert np.isfinite(got).all(), f"{what}: non-finite {name}"
    err = np.abs(got - ref)
    tol = 2.0 * bound + 1e-6 * np.abs(ref).max(initial=0.0)
    if bf16_out:
        tol = tol + bf16_half_ulp(np.abs(ref) + tol)
    bad = err > tol
    assert not bad.any(), (f"{what}: {name} max-abs {err.max():.3e}, worst excess "
                           f"{(err - tol).max():.3e} at {np.argwhere(bad)[:3].tolist()}")
    return float((err / np.maximum(tol, 1e-30)).max(initial=0.0))


def oracle_forward_inputs(q, k, v, scale, causal, cu_q=None, cu_k=None):
    """The oracle's O rounded to bf16 bits and its LSE rounded to fp32, plus
    both as fp64 for the bound."""
    if cu_q is None:
        o, lse = oracle.attention(q, k, v, scale, causal)
    else:
        o, lse = oracle.attention_varlen(q, k, v, cu_q, cu_k, scale, causal)
    o_bits = bf16_bits_of(o)
    lse32 = lse.astype(np.float32)
    return o_bits, lse32, W.bf16_bits_to_f32(o_bits).astype(np.float64), lse32.astype(np.float64)
