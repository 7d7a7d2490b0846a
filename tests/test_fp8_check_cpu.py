"""CPU check of the FP8 parity criterion (tests/test_gpu_fp8.py::check): an
admissible result (the oracle's reference rounding of P) passes, and results
with a planted mistake fail: a dropped key, keys shifted by one, a wrong V
descale, a wrong score scale."""
import numpy as np
import pytest

import oracle.fp8 as F
import workloads as W
from test_gpu_fp8 import check


@pytest.fixture(scope="module")
def case():
    q8, k8, v8, ds = W.make_fixed_fp8(1, 2, 1, 200, 256, 128, seed=40, wid=231)
    scale = 1 / np.sqrt(128)
    o_ex, l_ex = F.attention_fp8(q8, k8, v8, *ds, scale=scale, causal=True)
    return q8, k8, v8, ds, scale, o_ex, l_ex


def run(case, o, lse):
    q8, k8, v8, ds, scale, _, _ = case
    check(o, lse, q8, k8, v8, ds, scale, True, False, "cpu")


def test_reference_rounding_passes(case):
    q8, k8, v8, ds, scale, _, l_ex = case
    ref = F.attention_fp8_rounded_p(q8, k8, v8, *ds, scale=scale, causal=True)
    run(case, ref, l_ex)


def test_dropped_key_fails(case):
    """Attention over every admissible key but key 100 (the LSE kept exact)."""
    q8, k8, v8, ds, scale, _, l_ex = case
    q, k, v = (F.dequantize(x, d) for x, d in zip((q8, k8, v8), ds))
    lq, lk = q.shape[1], k.shape[1]
    o = np.zeros(q.shape)
    keep = np.ones(lk, bool)
    keep[100] = False
    for h in range(q.shape[2]):
        s = scale * q[0, :, h] @ k[0, :, 0].T
        adm = np.arange(lk)[None, :] <= np.arange(lq)[:, None] + (lk - lq)
        s = np.where(adm & keep[None, :], s, -np.inf)
        w = np.exp(s - s.max(axis=1, keepdims=True))
        o[0, :, h] = w @ v[0, :, 0] / w.sum(axis=1)[:, None]
    with pytest.raises(AssertionError):
        run(case, o, l_ex)


def test_shifted_keys_fail(case):
    q8, k8, v8, ds, scale, _, l_ex = case
    vs = np.roll(v8, 1, axis=1)
    o, _ = F.attention_fp8(q8, k8, vs, *ds, scale=scale, causal=True)
    with pytest.raises(AssertionError):
        run(case, o, l_ex)


def test_wrong_v_descale_fails(case):
    _, _, _, _, _, o_ex, l_ex = case
    with pytest.raises(AssertionError):
        run(case, o_ex * 1.05, l_ex)


def test_wrong_score_scale_fails(case):
    q8, k8, v8, ds, scale, _, _ = case
    o, l = F.attention_fp8(q8, k8, v8, *ds, scale=scale * 1.01, causal=True)
    with pytest.raises(AssertionError):
        run(case, o, l)
