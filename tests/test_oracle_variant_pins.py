"""Pins of the score-variant oracle (oracle/variants.py: sliding window,
ALiBi, softcap), each independent of the oracle's own code: reductions to the
plain oracle, per-row key slices, and closed forms (two keys under a softcap,
geometric ALiBi weights for equal raw scores, a one-key window)."""
import numpy as np
import pytest

import oracle
import oracle.variants as V
import workloads as W


def inputs(b, nq, nk, hq, hkv, d, seed):
    return W.make_fixed(b, hq, hkv, nq, nk, d, seed=seed, wid=401, k_mult=1.5)


def f64(x):
    return W.bf16_bits_to_f32(x).astype(np.float64)


@pytest.mark.parametrize("causal", [False, True])
def test_no_variant_is_the_plain_oracle(causal):
    q, k, v = inputs(2, 40, 55, 4, 2, 16, 1)
    o, l = V.attention_ext(q, k, v, 0.3, causal)
    o2, l2 = oracle.attention(q, k, v, 0.3, causal)
    assert np.array_equal(o, o2) and np.array_equal(l, l2)


def test_right_window_zero_is_causal():
    q, k, v = inputs(1, 30, 45, 2, 2, 16, 2)
    o, l = V.attention_ext(q, k, v, 0.3, False, window=(-1, 0))
    o2, l2 = oracle.attention(q, k, v, 0.3, True)
    assert np.array_equal(o, o2) and np.array_equal(l, l2)


@pytest.mark.parametrize("window,causal", [((3, 5), False), ((7, 0), False), ((0, 0), False),
                                           ((10, -1), True), ((-1, 4), False), ((2, 9), True)])
@pytest.mark.parametrize("nq,nk", [(20, 20), (12, 30), (30, 12)])
def test_window_equals_attention_on_each_rows_key_slice(window, causal, nq, nk):
    q, k, v = inputs(1, nq, nk, 1, 1, 16, 3)
    o, l = V.attention_ext(q, k, v, 0.25, causal, window=window)
    qf, kf, vf = f64(q)[0, :, 0], f64(k)[0, :, 0], f64(v)[0, :, 0]
    left, right = window
    for i in range(nq):
        c = i + nk - nq
        lo = 0 if left < 0 else max(0, c - left)
        hi = nk - 1 if right < 0 else min(nk - 1, c + right)
        if causal:
            hi = min(hi, c)
        if hi < lo:
            assert np.all(o[0, i, 0] == 0) and l[0, i, 0] == -np.inf
            continue
        s = 0.25 * kf[lo:hi + 1] @ qf[i]
        w = np.exp(s - s.max())
        np.testing.assert_allclose(o[0, i, 0], w @ vf[lo:hi + 1] / w.sum(), rtol=0, atol=1e-12)
        assert l[0, i, 0] == pytest.approx(s.max() + np.log(w.sum()), abs=1e-12)


def test_one_key_window_returns_that_value():
    q, k, v = inputs(1, 16, 16, 2, 1, 16, 4)
    o, l = V.attention_ext(q, k, v, 0.5, False, window=(0, 0))
    vf, qf, kf = f64(v), f64(q), f64(k)
    for h in range(2):
        np.testing.assert_allclose(o[0, :, h], vf[0, :, 0], rtol=0, atol=1e-13)
        np.testing.assert_allclose(l[0, :, h], 0.5 * np.sum(qf[0, :, h] * kf[0, :, 0], axis=1),
                                   rtol=0, atol=1e-12)


def test_softcap_two_keys_closed_form():
    rng = np.random.default_rng(5)
    for cap in (0.5, 2.0, 30.0):
        q = rng.standard_normal((1, 1, 1, 8)) * 2
        k = rng.standard_normal((1, 2, 1, 8)) * 2
        v = rng.standard_normal((1, 2, 1, 8))
        o, l = V.attention_ext(q, k, v, 0.7, False, softcap=cap)
        x1, x2 = (cap * np.tanh(0.7 * (q[0, 0, 0] @ k[0, j, 0]) / cap) for j in range(2))
        p1 = 1.0 / (1.0 + np.exp(x2 - x1))          # a logistic of the capped difference
        np.testing.assert_allclose(o[0, 0, 0], p1 * v[0, 0, 0] + (1 - p1) * v[0, 1, 0],
                                   rtol=0, atol=1e-13)
        assert l[0, 0, 0] == pytest.approx(np.logaddexp(x1, x2), abs=1e-13)


def test_softcap_limits():
    q, k, v = inputs(1, 25, 25, 2, 2, 16, 6)
    o, l = V.attention_ext(q, k, v, 0.4, True, softcap=1e7)
    o2, l2 = oracle.attention(q, k, v, 0.4, True)
    np.testing.assert_allclose(o, o2, rtol=0, atol=1e-9)
    np.testing.assert_allclose(l, l2, rtol=0, atol=1e-9)
    # a small cap bounds every score: LSE <= cap + ln(#keys)
    o, l = V.attention_ext(q, k, v, 0.4, False, softcap=0.3)
    assert np.all(l <= 0.3 + np.log(25) + 1e-12) and np.all(l >= -0.3 + np.log(25) - 1e-12)


@pytest.mark.parametrize("nq,nk", [(10, 10), (6, 14)])
def test_alibi_geometric_weights_for_equal_scores(nq, nk):
    """q = 0 makes every raw score 0; under causal ALiBi the weights of row i
    are r^dist, r = exp(-m), dist = i + delta - j = 0, 1, ..., so the row sum
    is the geometric series (1 - r^n) / (1 - r) over its n keys."""
    m = 0.37
    q = np.zeros((1, nq, 1, 8))
    rng = np.random.default_rng(7)
    k, v = rng.standard_normal((1, nk, 1, 8)), rng.standard_normal((1, nk, 1, 8))
    o, l = V.attention_ext(q, k, v, 1.0, True, alibi=np.array([m]))
    r = np.exp(-m)
    for i in range(nq):
        n = i + nk - nq + 1                      # keys 0 .. i + delta
        w = r ** np.arange(n)[::-1]              # key j has weight r^(i + delta - j)
        total = (1 - r ** n) / (1 - r)
        assert l[0, i, 0] == pytest.approx(np.log(total), abs=1e-13)
        np.testing.assert_allclose(o[0, i, 0], w @ v[0, :n, 0] / total, rtol=0, atol=1e-13)


def test_alibi_zero_slope_and_per_batch_slopes():
    q, k, v = inputs(2, 20, 30, 4, 2, 16, 8)
    o, l = V.attention_ext(q, k, v, 0.3, False, alibi=np.zeros(4))
    o2, l2 = oracle.attention(q, k, v, 0.3, False)
    assert np.array_equal(o, o2) and np.array_equal(l, l2)
    slopes = 2.0 ** (-np.arange(1, 5))
    ob, lb = V.attention_ext(q, k, v, 0.3, True, alibi=np.stack([slopes, slopes]))
    oh, lh = V.attention_ext(q, k, v, 0.3, True, alibi=slopes)
    assert np.array_equal(ob, oh) and np.array_equal(lb, lh)


def test_varlen_equals_separate_calls():
    lens = [7, 0, 33, 18]
    q, k, v, cu_q, cu_k = W.make_varlen(lens, lens, 4, 2, 16, seed=9, wid=402)
    slopes = np.array([[0.1, 0.2, 0.3, 0.4]] * 4) * np.arange(1, 5)[:, None]
    o, l = V.attention_ext_varlen(q, k, v, cu_q, cu_k, 0.3, True, window=(5, -1), softcap=4.0,
                                  alibi=slopes)
    for s in range(4):
        a, b = cu_q[s], cu_q[s + 1]
        os_, ls = V.attention_ext(q[None, a:b], k[None, a:b], v[None, a:b], 0.3, True,
                                  window=(5, -1), softcap=4.0, alibi=slopes[s])
        assert np.array_equal(o[a:b], os_[0]) and np.array_equal(l[a:b], ls[0])


def test_softcap_then_alibi_two_keys_closed_form():
    """One query, two keys, causal: the cap applies to the scaled score and
    the distance bias (1 for the first key, 0 for the last) comes after it."""
    rng = np.random.default_rng(10)
    q = rng.standard_normal((1, 1, 1, 8)) * 3
    k = rng.standard_normal((1, 2, 1, 8)) * 3
    v = rng.standard_normal((1, 2, 1, 8))
    cap, m = 1.5, 0.8
    o, l = V.attention_ext(q, k, v, 0.6, True, softcap=cap, alibi=np.array([m]))
    s0, s1 = (0.6 * (q[0, 0, 0] @ k[0, j, 0]) for j in range(2))
    x0, x1 = cap * np.tanh(s0 / cap) - m, cap * np.tanh(s1 / cap)
    p0 = 1.0 / (1.0 + np.exp(x1 - x0))
    np.testing.assert_allclose(o[0, 0, 0], p0 * v[0, 0, 0] + (1 - p0) * v[0, 1, 0], rtol=0,
                               atol=1e-13)
    assert l[0, 0, 0] == pytest.approx(np.logaddexp(x0, x1), abs=1e-13)
