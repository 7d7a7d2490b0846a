"""Plant plausible mistakes in the score-variant oracle (on the CPU) and check
that the pins of tests/test_oracle_variant_pins.py catch every one."""
import numpy as np
import pytest

import oracle.variants as V
import test_oracle_variant_pins as P
from test_oracle_kvcache_mutants import run_all_pins as _run

ORIG_SCORES = V.variant_scores
ORIG_MASK = V.window_mask


def _window_off_by_one(lq, lk, causal, left, right):
    return ORIG_MASK(lq, lk, causal, left + 1 if left >= 0 else left, right)


def _window_top_left(lq, lk, causal, left, right):
    # forgets the bottom-right alignment of the window
    i = np.arange(lq)[:, None]
    j = np.arange(lk)[None, :]
    m = np.ones((lq, lk), dtype=bool)
    if left >= 0:
        m &= j >= i - left
    if right >= 0:
        m &= j <= i + right
    if causal:
        m &= j <= i + (lk - lq)
    return m


def _alibi_sign(qh, kh, scale, softcap, slope):
    return ORIG_SCORES(qh, kh, scale, softcap, -slope)


def _alibi_no_delta(qh, kh, scale, softcap, slope):
    lq, lk = qh.shape[0], kh.shape[0]
    x = ORIG_SCORES(qh, kh, scale, softcap, 0.0)
    if slope:
        x = x - slope * np.abs(np.arange(lq)[:, None] - np.arange(lk)[None, :])
    return x


def _softcap_without_outer_factor(qh, kh, scale, softcap, slope):
    x = scale * (qh @ kh.T)
    if softcap > 0:
        x = np.tanh(x / softcap)
    lq, lk = x.shape
    if slope:
        x = x - slope * np.abs(np.arange(lq)[:, None] + (lk - lq) - np.arange(lk)[None, :])
    return x


def _softcap_after_alibi(qh, kh, scale, softcap, slope):
    x = ORIG_SCORES(qh, kh, scale, 0.0, slope)
    return softcap * np.tanh(x / softcap) if softcap > 0 else x


MUTANTS = {
    "window off by one": ("window_mask", _window_off_by_one),
    "window not bottom-right aligned": ("window_mask", _window_top_left),
    "ALiBi sign": ("variant_scores", _alibi_sign),
    "ALiBi distance without delta": ("variant_scores", _alibi_no_delta),
    "softcap missing its factor": ("variant_scores", _softcap_without_outer_factor),
    "softcap after ALiBi": ("variant_scores", _softcap_after_alibi),
}


def run_all_pins():
    import test_oracle_kvcache_mutants as KM
    saved = KM.PINS
    KM.PINS = [getattr(P, n) for n in dir(P) if n.startswith("test_")]
    try:
        return _run()
    finally:
        KM.PINS = saved


def test_pins_pass_unmutated():
    assert run_all_pins() == 0


@pytest.mark.parametrize("name", list(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(V, attr, fn)
    assert run_all_pins() >= 1, name
