"""fp64 CPU oracle for the FP8 attention forward.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module.  The HIP
library never routes through it and shares no code with it.

The first page's FlashAttention 3 notes ("推理优化 | FlashAttention 1-4 详解",
section FlashAttention 3 的硬件特性利用, the low-precision item, and the
summary table's FA3 column) say only that the forward runs its matrix
products on FP8 matrix units while the backward stays in BF16.  The readings
taken where the page is silent:

  * Q, K and V arrive as FP8 E4M3 codes with one fp32 descale per tensor: the
    real tensor is descale times the decoded codes.  E4M3 here is the OCP
    8-bit float: 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits; an
    exponent field of 0 encodes subnormals m/8 * 2^-6; the all-ones pattern
    S.1111.111 is NaN; there are no infinities; the largest finite value is
    448.
  * The result is exact attention (``oracle.exact``) of the real tensors:
    O and the natural-log LSE of scale * <dq q_i, dk k_j>.
  * Both products run on FP8, so the probabilities are rounded to E4M3
    before they meet V.  That rounding is an approximation step of the
    method, not part of the definition: ``p_rounding_bound`` bounds its
    effect on O, and ``attention_fp8_rounded_p`` takes the step once, with
    the probabilities relative to each row's maximum, as a reference for the
    size of the error the step makes.
"""
from __future__ import annotations

import numpy as np

from .exact import _group, admissible_mask, attention, kv_head

E4M3_MAX = 448.0
E4M3_MIN_NORMAL = 2.0 ** -6
E4M3_SUBNORMAL_STEP = 2.0 ** -9


def e4m3_to_f64(codes) -> np.ndarray:
    """Decode E4M3 codes (uint8) to float64 from the field definition."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c >> 7, -1.0, 1.0)
    e = (c >> 3) & 15
    m = (c & 7).astype(np.float64)
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & ((c & 7) == 7), np.nan, mag)
    return sign * mag


def round_to_e4m3(x) -> np.ndarray:
    """Round float64 values of magnitude <= 448 to the nearest E4M3 value
    (ties to the even mantissa), returned as float64.  Spacing in [2^e,
    2^(e+1)) is 2^(e-3) for e >= -6; below 2^-6 it is the subnormal step
    2^-9."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    if np.any(a > E4M3_MAX):
        raise ValueError("value outside the E4M3 range")
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, -6.0)
    step = np.exp2(e - 3.0)
    q = a / step                       # exact: step is a power of two
    r = np.floor(q)
    frac = q - r
    up = (frac > 0.5) | ((frac == 0.5) & (np.mod(r, 2.0) == 1.0))
    r = r + up
    return np.sign(x) * r * step


def dequantize(codes, descale: float) -> np.ndarray:
    """descale (an fp32 value) times the decoded codes."""
    return np.float64(np.float32(descale)) * e4m3_to_f64(codes)


def attention_fp8(q8, k8, v8, q_descale, k_descale, v_descale, scale: float,
                  causal: bool = False):
    """Fixed-length batch of E4M3 codes: q8 [B, Nq, Hq, d], k8/v8 [B, Nk, Hkv, d].
    Exact attention of the dequantised tensors: (O [B, Nq, Hq, d], LSE [B, Nq, Hq])."""
    return attention(dequantize(q8, q_descale), dequantize(k8, k_descale),
                     dequantize(v8, v_descale), scale, causal)


def _head_terms(qh, kh, scale, causal):
    """Normalised weights w = exp(s - m) (1 at each row's maximum) and their
    row sums, over the admissible keys of one (sequence, head)."""
    lq, lk = qh.shape[0], kh.shape[0]
    s = scale * (qh @ kh.T)
    mask = admissible_mask(np.arange(lq), lq, lk, causal)
    s = np.where(mask, s, -np.inf)
    m = s.max(axis=1, keepdims=True)
    m = np.where(np.isfinite(m), m, 0.0)
    w = np.exp(s - m)
    return w, w.sum(axis=1)


def p_rounding_bound(q8, k8, v8, q_descale, k_descale, v_descale, scale: float,
                     causal: bool = False) -> np.ndarray:
    """Elementwise bound [B, Nq, Hq, d] on |O_fp8 - O_exact| from rounding the
    probabilities to E4M3 before the P V product.

    A kernel scales each probability by 2^t for some t >= 0 (its running
    reference lies at or below the row maximum) before rounding, so the
    rounded value w~ of a weight w = exp(s - m) <= 1 satisfies
    |w~ - w| <= 2^-4 w + min(w, 2^-10): half a unit in the last place of a
    normal E4M3 value (3 mantissa bits), plus half the subnormal step 2^-9,
    which scaling up by 2^t only shrinks.  With the row sum taken over the
    unrounded weights, |dO_id| <= sum_j |w~_j - w_j| |v_jd| / sum_j w_j."""
    q = dequantize(q8, q_descale)
    k = dequantize(k8, k_descale)
    v = dequantize(v8, v_descale)
    bsz, nq, hq, d = q.shape
    g = _group(hq, k.shape[2])
    out = np.zeros((bsz, nq, hq, d))
    for b in range(bsz):
        for h in range(hq):
            kh = kv_head(h, g)
            w, l = _head_terms(q[b, :, h], k[b, :, kh], scale, causal)
            dw = 2.0 ** -4 * w + np.minimum(w, 2.0 ** -10)
            ok = l > 0
            out[b, ok, h] = (dw[ok] @ np.abs(v[b, :, kh])) / l[ok][:, None]
    return out


def attention_fp8_rounded_p(q8, k8, v8, q_descale, k_descale, v_descale, scale: float,
                            causal: bool = False):
    """O [B, Nq, Hq, d] with the probabilities exp(s - m) (relative to each
    row's maximum) rounded to E4M3 before the product with V and the row sum
    over the unrounded ones: one admissible instance of the FP8 method's
    rounding step, whose distance from the exact O sets the scale of the
    error a kernel may make."""
    q = dequantize(q8, q_descale)
    k = dequantize(k8, k_descale)
    v = dequantize(v8, v_descale)
    bsz, nq, hq, d = q.shape
    g = _group(hq, k.shape[2])
    out = np.zeros((bsz, nq, hq, d))
    for b in range(bsz):
        for h in range(hq):
            kh = kv_head(h, g)
            w, l = _head_terms(q[b, :, h], k[b, :, kh], scale, causal)
            ok = l > 0
            out[b, ok, h] = (round_to_e4m3(w[ok]) @ v[b, :, kh]) / l[ok][:, None]
    return out
