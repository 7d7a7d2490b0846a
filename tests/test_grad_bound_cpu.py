"""The backward tests' tolerance, checked on the CPU.

A plain fp64 emulation of the backward's arithmetic (P and dS rounded to
bf16 before their products, D taken from the bf16 O) must pass the bound of
``_grad_bounds`` with room to spare, and the kernel mistakes one would expect
(a dropped key block, the diagonal masked out, D left at zero, a missing
scale, grouped heads summed into the wrong kv head, dS taken from the
unnormalised row) must each fail it.  The emulation and its mutants live in
this file only; they share nothing with the HIP library.
"""
import numpy as np
import pytest

import oracle
import workloads as W
from _grad_bounds import check_grad, fixed_bounds, oracle_forward_inputs


def bf(x):
    bits = W.round_f32_to_bf16_bits(np.asarray(x, np.float32))
    return W.bf16_bits_to_f32(bits).astype(np.float64)


def emulate(q, k, v, do, o_in, lse_in, scale, causal, mutant=None):
    q, k, v, do = (W.bf16_bits_to_f32(x).astype(np.float64) for x in (q, k, v, do))
    dq, dk, dv = np.zeros(q.shape), np.zeros(k.shape), np.zeros(v.shape)
    g = q.shape[2] // k.shape[2]
    for b in range(q.shape[0]):
        for h in range(q.shape[2]):
            kv = h // g
            if mutant == "gqa_head" and g > 1:
                kv = h % k.shape[2]
            qh, kh, vh, doh = q[b, :, h], k[b, :, kv], v[b, :, kv], do[b, :, h]
            lq, lk = qh.shape[0], kh.shape[0]
            mask = oracle.admissible_mask(np.arange(lq), lq, lk, causal)
            if mutant == "diagonal" and causal:
                mask = mask & ~np.eye(lq, lk, k=lk - lq, dtype=bool)
            if mutant == "key_block":
                mask[:, 32:64] = False
            lse = lse_in[b, :, h]
            fin = np.isfinite(lse)
            s = scale * (qh @ kh.T)
            p = np.where(mask & fin[:, None],
                         np.exp(np.where(mask, s, 0.0) - np.where(fin, lse, 0.0)[:, None]), 0.0)
            dsum = (doh * o_in[b, :, h]).sum(axis=1)
            if mutant == "no_dsum":
                dsum = np.zeros_like(dsum)
            ds = p * (doh @ vh.T - dsum[:, None])
            sc = 1.0 if mutant == "no_scale" else scale
            dq[b, :, h] = scale * (bf(ds) @ kh)
            dk[b, :, h // g] += sc * (bf(ds).T @ qh)
            dv[b, :, h // g] += bf(p).T @ doh
    return dq, dk, dv


CASES = [(1, 150, 150, 2, 1, 64, True), (1, 90, 130, 4, 2, 128, False)]


def setup(case):
    bsz, nq, nk, hq, hkv, d, causal = case
    q, k, v = W.make_fixed(bsz, hq, hkv, nq, nk, d, seed=21, wid=301, k_mult=1.5)
    do = W.make_dout(q.shape, seed=21, wid=301)
    scale = 1.0 / np.sqrt(d)
    _, _, o_in, lse_in = oracle_forward_inputs(q, k, v, scale, causal)
    ref = oracle.attention_grad(q, k, v, do, scale, causal)
    bnd = fixed_bounds(q, k, v, do, o_in, lse_in, scale, causal)
    return q, k, v, do, o_in, lse_in, scale, causal, ref, bnd


@pytest.mark.parametrize("case", CASES, ids=[str(c) for c in CASES])
def test_faithful_emulation_passes_with_margin(case):
    q, k, v, do, o_in, lse_in, scale, causal, ref, bnd = setup(case)
    got = emulate(q, k, v, do, o_in, lse_in, scale, causal)
    for name, g, r, b in zip(("dQ", "dK", "dV"), got, ref, bnd):
        # check_grad returns err / tolerance at its worst element
        assert check_grad(name, g, r, b, False, str(case)) < 0.75


@pytest.mark.parametrize("mutant", ["diagonal", "key_block", "no_dsum", "no_scale",
                                    "gqa_head"])
def test_planted_mistakes_fail_the_bound(mutant):
    case = CASES[0] if mutant == "diagonal" else CASES[1]
    q, k, v, do, o_in, lse_in, scale, causal, ref, bnd = setup(case)
    got = emulate(q, k, v, do, o_in, lse_in, scale, causal, mutant)
    failed = 0
    for name, g, r, b in zip(("dQ", "dK", "dV"), got, ref, bnd):
        try:
            check_grad(name, g, r, b, False, mutant)
        except AssertionError:
            failed += 1
    assert failed >= 1, mutant
