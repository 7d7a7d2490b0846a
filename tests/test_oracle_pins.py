"""Pins of the fp64 oracle to facts fixed outside it (CPU only).

Each ``pin_*`` function checks the oracle against something other than
itself: hand-worked examples (tests/golden), closed forms, invariants of the
definition, library routines (scipy's logsumexp/softmax, torch's CPU
scaled_dot_product_attention in float64), and a second algorithm (the online
softmax recurrence of "推理优化 | FlashAttention 1-4 详解", §Online Softmax
数学推导).  ``tests/test_oracle_mutants.py`` plants plausible mistakes in the
oracle and checks that these pins catch each one.
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.special

import oracle
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")
TIGHT = 1e-12


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def _ref_mask(lq, lk, causal):
    i = np.arange(lq)[:, None]
    j = np.arange(lk)[None, :]
    return (j <= i + lk - lq) if causal else np.ones((lq, lk), bool)


# --------------------------------------------------------------------------
# pins
# --------------------------------------------------------------------------
def pin_worked_examples():
    """Hand-derived values of tiny cases (tests/golden/worked_examples.json)."""
    with open(GOLDEN) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        q, k, v = (np.array(c[x], np.float64) for x in "qkv")
        o, lse = oracle.head_attention(q, k, v, c["scale"], c["causal"])
        exp_o = np.array(c["expected_o"], np.float64)
        exp_l = np.array([float(x) for x in c["expected_lse"]])
        assert np.allclose(o, exp_o, rtol=0, atol=c["tol"]), (c["name"], o, exp_o)
        fin = np.isfinite(exp_l)
        assert np.array_equal(np.isfinite(lse), fin), (c["name"], lse)
        assert np.allclose(lse[fin], exp_l[fin], rtol=0, atol=c["tol"]), (c["name"], lse)


def pin_two_pass_equals_online_tiled():
    """The two-pass definition equals the tiled online-softmax recurrence for
    odd tile sizes, causal and not, Lq == Lk and Lq != Lk."""
    for (lq, lk, d, seed) in [(23, 23, 8, 1), (17, 40, 5, 2), (40, 17, 6, 3), (130, 131, 16, 4)]:
        q, k, v = _rand((lq, d), seed), _rand((lk, d), seed + 10, 2.0), _rand((lk, d), seed + 20)
        for causal in (False, True):
            o, l = oracle.head_attention(q, k, v, 0.37, causal)
            for br, bc in [(1, 1), (3, 7), (7, 3), (128, 128)]:
                ot, lt = oracle.tiled_online_attention(q, k, v, 0.37, br, bc, causal)
                fin = np.isfinite(l)
                assert np.array_equal(fin, np.isfinite(lt))
                assert np.abs(ot - o).max() <= TIGHT, (lq, lk, causal, br, bc)
                assert np.abs(lt[fin] - l[fin]).max(initial=0) <= TIGHT


def pin_lse_and_probabilities_match_scipy():
    """LSE equals scipy.special.logsumexp of the masked scaled scores, and with
    V = identity (Lk <= d) each output row is the softmax row, which sums to 1."""
    for (lq, lk, causal, seed) in [(9, 12, False, 5), (12, 12, True, 6), (5, 12, True, 7)]:
        d = 12
        q, k = _rand((lq, d), seed), _rand((lk, d), seed + 1)
        scale = 0.41
        s = scale * np.einsum("id,jd->ij", q, k)
        mask = _ref_mask(lq, lk, causal)
        s_masked = np.where(mask, s, -np.inf)
        o, lse = oracle.head_attention(q, k, np.eye(lk, d), scale, causal)
        assert np.abs(lse - scipy.special.logsumexp(s_masked, axis=1)).max() <= TIGHT
        p_ref = scipy.special.softmax(s_masked, axis=1)
        assert np.abs(o[:, :lk] - p_ref).max() <= TIGHT
        assert np.abs(o.sum(axis=1) - 1.0).max() <= TIGHT
        assert (o >= 0).all()


def pin_constant_v():
    """Constant V = c gives O = c for every admissible row, any mask."""
    for causal in (False, True):
        q, k = _rand((31, 8), 8, 3.0), _rand((29, 8), 9, 3.0)
        v = np.full((29, 8), -1.75)
        o, lse = oracle.head_attention(q, k, v, 0.9, causal)
        fin = np.isfinite(lse)
        assert np.abs(o[fin] + 1.75).max() <= TIGHT
        assert np.all(o[~fin] == 0)


def pin_equal_scores_give_means():
    """Q = 0 makes all scores equal: O is the mean of V over admissible keys and
    LSE = ln |admissible|; causal rows give prefix means."""
    lk, d = 37, 6
    v = _rand((lk, d), 11)
    for causal in (False, True):
        o, lse = oracle.head_attention(np.zeros((lk, d)), _rand((lk, d), 12), v, 0.5, causal)
        for i in range(lk):
            n = i + 1 if causal else lk
            assert np.abs(o[i] - v[:n].mean(axis=0)).max() <= TIGHT
            assert abs(lse[i] - math.log(n)) <= TIGHT


def pin_causal_row_zero():
    """Causal with Lq == Lk: row 0 sees key 0 only, so O = V[0] and
    LSE = scale * <q0, k0>."""
    q, k, v = _rand((20, 8), 13), _rand((20, 8), 14), _rand((20, 8), 15)
    o, lse = oracle.head_attention(q, k, v, 0.3, True)
    assert np.abs(o[0] - v[0]).max() <= TIGHT
    assert abs(lse[0] - 0.3 * float(q[0] @ k[0])) <= TIGHT


def pin_shift_invariance():
    """Adding a constant c to every score of a row leaves O unchanged and adds c
    to LSE (realised by an extra feature: q' = [q, 1], k' = [k, c/scale]).  With
    c = 800 an unshifted exp overflows."""
    q, k, v = _rand((11, 5), 16), _rand((13, 5), 17), _rand((13, 5), 18)
    scale, c = 0.6, 800.0
    o0, l0 = oracle.head_attention(q, k, v, scale, False)
    q2 = np.concatenate([q, np.ones((11, 1))], axis=1)
    k2 = np.concatenate([k, np.full((13, 1), c / scale)], axis=1)
    o1, l1 = oracle.head_attention(q2, k2, v, scale, False)
    assert np.abs(o1 - o0).max() <= 1e-10
    assert np.abs(l1 - (l0 + c)).max() <= 1e-10


def pin_torch_sdpa():
    """Cross-check with torch's CPU scaled_dot_product_attention in float64,
    batched, with GQA (K/V heads repeated), causal and not."""
    import torch
    for (bsz, lq, lk, hq, hkv, d, causal, seed) in [
            (2, 33, 33, 4, 2, 16, True, 19), (1, 7, 50, 6, 3, 8, False, 20),
            (2, 9, 21, 4, 1, 8, True, 21)]:
        q = _rand((bsz, lq, hq, d), seed)
        k = _rand((bsz, lk, hkv, d), seed + 1)
        v = _rand((bsz, lk, hkv, d), seed + 2)
        scale = 1.0 / math.sqrt(d)
        o, lse = oracle.attention(q, k, v, scale, causal)
        g = hq // hkv
        tq = torch.from_numpy(q).permute(0, 2, 1, 3)
        tk = torch.from_numpy(k).permute(0, 2, 1, 3).repeat_interleave(g, dim=1)
        tv = torch.from_numpy(v).permute(0, 2, 1, 3).repeat_interleave(g, dim=1)
        mask = torch.from_numpy(_ref_mask(lq, lk, causal))
        ref = torch.nn.functional.scaled_dot_product_attention(
            tq, tk, tv, attn_mask=mask, scale=scale).permute(0, 2, 1, 3).numpy()
        assert np.abs(o - ref).max() <= TIGHT, (bsz, lq, lk, causal)


def pin_gqa_equals_repeated_mha():
    """GQA equals MHA with each K/V head repeated for its group of query heads."""
    q = _rand((2, 15, 8, 8), 22)
    k, v = _rand((2, 17, 2, 8), 23), _rand((2, 17, 2, 8), 24)
    o, l = oracle.attention(q, k, v, 0.35, True)
    o2, l2 = oracle.attention(q, np.repeat(k, 4, axis=2), np.repeat(v, 4, axis=2), 0.35, True)
    assert np.abs(o - o2).max() == 0 and np.array_equal(l, l2)


def pin_varlen_equals_separate_sequences():
    """Packed sequences equal separate single-sequence calls."""
    lens_q, lens_k = [5, 1, 17, 9], [5, 3, 17, 12]
    q, k, v, cu_q, cu_k = W.make_varlen(lens_q, lens_k, 4, 2, 16, seed=3, wid=99)
    o, l = oracle.attention_varlen(q, k, v, cu_q, cu_k, 0.25, True)
    for s in range(4):
        qs = q[cu_q[s]:cu_q[s + 1]][None]
        ks, vs = k[cu_k[s]:cu_k[s + 1]][None], v[cu_k[s]:cu_k[s + 1]][None]
        os_, ls = oracle.attention(qs, ks, vs, 0.25, True)
        assert np.abs(o[cu_q[s]:cu_q[s + 1]] - os_[0]).max() == 0
        assert np.array_equal(l[cu_q[s]:cu_q[s + 1]], ls[0])


def pin_rows_equal_full():
    """Row-by-row evaluation equals the full evaluation (fixed and packed)."""
    q, k, v = W.make_fixed(2, 4, 2, 19, 23, 16, seed=4, wid=98)
    o, l = oracle.attention(q, k, v, 0.25, True)
    rows = [(0, 0, 0), (1, 18, 3), (1, 7, 2)]
    o2, l2 = oracle.attention_rows(q, k, v, rows, 0.25, True)
    for n, (b, i, h) in enumerate(rows):
        assert np.abs(o2[n] - o[b, i, h]).max() <= TIGHT and abs(l2[n] - l[b, i, h]) <= TIGHT


def pin_split_merge_invariance():
    """Attention over disjoint key parts, merged by LSE weight, equals attention
    over all keys (the block merge of the lecture notes, §6); an empty part
    (LSE = -inf, arbitrary O) has no effect."""
    q, k, v = _rand((6, 8), 25), _rand((50, 8), 26, 2.0), _rand((50, 8), 27)
    o, l = oracle.head_attention(q, k, v, 0.5, False)
    for cuts in ([0, 50], [0, 1, 50], [0, 13, 14, 40, 50], list(range(0, 51, 5))):
        parts = [oracle.head_attention(q, k[a:b], v[a:b], 0.5, False)
                 for a, b in zip(cuts[:-1], cuts[1:])]
        op = np.stack([p[0] for p in parts] + [np.full((6, 8), np.nan)], axis=1)
        lp = np.stack([p[1] for p in parts] + [np.full(6, -np.inf)], axis=1)
        om, lm = oracle.merge_partials(op, lp)
        assert np.abs(om - o).max() <= TIGHT and np.abs(lm - l).max() <= TIGHT
    om, lm = oracle.merge_partials(np.zeros((2, 3, 4)), np.full((2, 3), -np.inf))
    assert np.all(om == 0) and np.all(np.isneginf(lm))


def pin_decode_equals_prefix_attention():
    """Decode equals attention of one query against the valid cache prefix, and
    NaN rows past the prefix are never used."""
    lens = np.array([3, 40, 17], np.int32)
    q, k, v = W.make_decode(3, 8, 2, 48, 16, lens, seed=5, wid=97, tail="nan")
    o, l = oracle.decode(q, k, v, lens, 0.25)
    assert np.isfinite(o).all() and np.isfinite(l).all()
    for b in range(3):
        n = int(lens[b])
        ob, lb = oracle.attention(q[b][None, None], k[b:b + 1, :n], v[b:b + 1, :n], 0.25, True)
        assert np.abs(o[b] - ob[0, 0]).max() <= TIGHT and np.abs(l[b] - lb[0, 0]).max() <= TIGHT


def pin_fully_masked_rows():
    """Rows with no admissible key (bottom-right causal, Lq > Lk) give O = 0 and
    LSE = -inf; the rest match the same rows computed alone."""
    q, k, v = _rand((9, 4), 28), _rand((4, 4), 29), _rand((4, 4), 30)
    o, l = oracle.head_attention(q, k, v, 1.0, True)
    assert np.all(o[:5] == 0) and np.all(np.isneginf(l[:5]))
    for i in range(5, 9):
        n = i - 4
        oi, li = oracle.head_attention(q[i:i + 1], k[:n], v[:n], 1.0, False)
        assert np.abs(o[i] - oi[0]).max() <= TIGHT and abs(l[i] - li[0]) <= TIGHT


PINS = [pin_worked_examples, pin_two_pass_equals_online_tiled,
        pin_lse_and_probabilities_match_scipy, pin_constant_v, pin_equal_scores_give_means,
        pin_causal_row_zero, pin_shift_invariance, pin_torch_sdpa, pin_gqa_equals_repeated_mha,
        pin_varlen_equals_separate_sequences, pin_rows_equal_full, pin_split_merge_invariance,
        pin_decode_equals_prefix_attention, pin_fully_masked_rows]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin()


def test_bf16_widening_is_exact():
    """The oracle widens bf16 bit patterns exactly (every finite pattern)."""
    bits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    with np.errstate(invalid="ignore"):
        f = oracle.to_f64(bits)
    fin = np.isfinite(f)
    back = (f[fin].astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal(back, bits[fin])
