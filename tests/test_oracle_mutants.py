"""Plant plausible mistakes in the oracle (on the CPU) and check that the pins
of tests/test_oracle_pins.py catch every one of them."""
import numpy as np
import pytest

import oracle.exact as OA
from test_oracle_pins import PINS


def _no_scale(qh, kh, scale):
    return qh @ kh.T


def _transposed_scores(qh, kh, scale):
    # K Q^T instead of Q K^T; only shape-compatible when square, so fall back
    # to the right product otherwise (the mistake then hides on non-square
    # cases and must be caught by a square one).
    if qh.shape[0] == kh.shape[0]:
        return scale * (kh @ qh.T)
    return scale * (qh @ kh.T)


def _mask_off_by_one(row_ids, lq, lk, causal):
    j = np.arange(lk)[None, :]
    if not causal:
        return np.ones((len(row_ids), lk), dtype=bool)
    return j < (np.asarray(row_ids)[:, None] + (lk - lq))


def _mask_top_left(row_ids, lq, lk, causal):
    j = np.arange(lk)[None, :]
    if not causal:
        return np.ones((len(row_ids), lk), dtype=bool)
    return j <= np.asarray(row_ids)[:, None]


def _softmax_no_shift(s, mask):
    s = np.where(mask, s, -np.inf)
    with np.errstate(over="ignore", invalid="ignore"):
        p = np.where(mask, np.exp(s), 0.0)
    l = p.sum(axis=1)
    m = np.zeros(s.shape[0])
    return p, m, l


def _softmax_sign(s, mask):
    s = np.where(mask, s, -np.inf)
    m = s.max(axis=1)
    shift = np.where(np.isfinite(m), m, 0.0)
    p = np.where(mask, np.exp(shift[:, None] - s), 0.0)
    return p, m, p.sum(axis=1)


def _kv_head_modulo(h, group):
    # interleaved instead of consecutive grouping
    return h % max(1, group) if group > 1 else h


def _weighted_transposed(p, vh, l):
    if p.shape[0] == p.shape[1]:
        return (p.T @ vh) / l[:, None]
    return (p @ vh) / l[:, None]


def _weighted_unnormalised(p, vh, l):
    return p @ vh


MUTANTS = {
    "scale_dropped": ("scores", _no_scale),
    "scores_transposed": ("scores", _transposed_scores),
    "causal_off_by_one": ("admissible_mask", _mask_off_by_one),
    "causal_top_left": ("admissible_mask", _mask_top_left),
    "softmax_without_max_shift": ("softmax_rows", _softmax_no_shift),
    "softmax_sign_flipped": ("softmax_rows", _softmax_sign),
    "gqa_interleaved": ("kv_head", _kv_head_modulo),
    "pv_transposed": ("weighted_values", _weighted_transposed),
    "missing_normalisation": ("weighted_values", _weighted_unnormalised),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(OA, attr, fn)
    caught = []
    for pin in PINS:
        try:
            with np.errstate(all="ignore"):
                pin()
        except (AssertionError, ValueError, FloatingPointError, IndexError):
            caught.append(pin.__name__)
    assert caught, f"no pin catches the planted mistake {name}"


def test_merge_mutant_caught(monkeypatch):
    """An unnormalised merge (weights exp(LSE_s) without the max shift and the
    division by their sum) is caught by the split-merge pin."""
    from test_oracle_pins import pin_split_merge_invariance

    def bad_merge(o_parts, lse_parts):
        w = np.exp(np.asarray(lse_parts))
        o = (w[..., None] * np.nan_to_num(np.asarray(o_parts))).sum(axis=-2)
        return o, np.log(w.sum(axis=-1))

    monkeypatch.setattr(OA, "merge_partials", bad_merge)
    import oracle
    monkeypatch.setattr(oracle, "merge_partials", bad_merge)
    with pytest.raises(AssertionError):
        with np.errstate(all="ignore"):
            pin_split_merge_invariance()
