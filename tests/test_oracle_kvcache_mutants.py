"""Plant plausible mistakes in the KV-cache step oracle (on the CPU) and check
that the pins of tests/test_oracle_kvcache_pins.py catch every one."""
import numpy as np
import pytest

import oracle.kvcache as KV
import test_oracle_kvcache_pins as P

ORIG_ROTARY = KV.rotary
ORIG_STEP = KV.kvcache_step
ORIG_INDEX = KV.cache_row_index


def _sin_flipped(x, cos_t, sin_t, rotary_dim, interleaved=False):
    return ORIG_ROTARY(x, cos_t, -np.asarray(sin_t), rotary_dim, interleaved)


def _pairs_swapped(x, cos_t, sin_t, rotary_dim, interleaved=False):
    return ORIG_ROTARY(x, cos_t, sin_t, rotary_dim, not interleaved)


def _position_off_by_one(q, k_cache, v_cache, cache_seqlens, scale, **kw):
    cos, sin = kw.get("rotary_cos"), kw.get("rotary_sin")
    if cos is not None:
        kw = dict(kw, rotary_cos=np.roll(cos, -1, axis=0), rotary_sin=np.roll(sin, -1, axis=0))
    return ORIG_STEP(q, k_cache, v_cache, cache_seqlens, scale, **kw)


def _new_key_not_attended(q, k_cache, v_cache, cache_seqlens, scale, **kw):
    o, l, k2, v2 = ORIG_STEP(q, k_cache, v_cache, cache_seqlens, scale, **kw)
    if kw.get("k_new") is None:
        return o, l, k2, v2
    o2, l2, _, _ = ORIG_STEP(q, k2, v2, cache_seqlens, scale,
                             **{a: b for a, b in kw.items() if a not in ("k_new", "v_new")})
    return o2, l2, k2, v2


def _page_row_swapped(b, j, block_table, page_size):
    if block_table is None:
        return b, j
    return int(block_table[b][j % len(block_table[b])]), j // len(block_table[b])


def _no_rounding(x):
    return np.asarray(x, np.float64)


MUTANTS = {
    "sin sign flipped": ("rotary", _sin_flipped),
    "pair layout swapped": ("rotary", _pairs_swapped),
    "rotary at position t+1": ("kvcache_step", _position_off_by_one),
    "appended key not attended": ("kvcache_step", _new_key_not_attended),
    "page and row swapped": ("cache_row_index", _page_row_swapped),
    "rotated values not rounded": ("to_bf16_rne", _no_rounding),
}

PINS = [getattr(P, n) for n in dir(P) if n.startswith("test_")]


def run_all_pins():
    failures = 0
    for pin in PINS:
        params = getattr(pin, "pytestmark", [])
        combos = [{}]
        for m in params:
            if m.name == "parametrize":
                names = [a.strip() for a in m.args[0].split(",")]
                combos = [dict(c, **dict(zip(names, v if len(names) > 1 else (v,))))
                          for c in combos for v in m.args[1]]
        for kw in combos:
            try:
                pin(**kw)
            except AssertionError:
                failures += 1
    return failures


def test_pins_pass_unmutated():
    assert run_all_pins() == 0


@pytest.mark.parametrize("name", list(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(KV, attr, fn)
    assert run_all_pins() >= 1, name
