"""Seeded random shapes through the forward, packed-batch, score-variant,
split-KV decode and FP8 entry points, each compared with the fp64 oracle
through the C ABI (needs a GPU).

The shapes are drawn once from fixed seeds (numpy PCG64), so the case list is
the same on every run and every case has its own test id.  They mix ragged
lengths (tails of 1 to 63 rows past a tile), query/key length mismatches,
empty sequences, grouped heads, both head dims, both output types and, for a
few cases, lengths long enough for the 256-row prefill workgroups.  Bounds are
those of the fixed-case tests: max-abs 1e-2 on O (fp32 O; bf16 O adds half a
bf16 ulp of the exact value), 1e-3 on the natural-log LSE, the same -inf rows;
the FP8 cases use the bound of test_gpu_fp8.check."""
import numpy as np
import pytest

import oracle
import oracle.variants as V
import workloads as W
from _gpu_helpers import check_lse, check_o, dev_bf16, dev_i32, host, say

pytestmark = pytest.mark.gpu
WID = 250


def _fixed_cases():
    rng = np.random.default_rng(20261202)
    cases = []
    for i in range(18):
        long_case = i >= 15                       # 256-row workgroups (Nq >= 1024, d = 128)
        b = 1 if long_case else int(rng.integers(1, 4))
        nq = int(rng.integers(2048, 2600)) if long_case else int(rng.integers(1, 700))
        nk = nq if rng.random() < 0.6 else int(rng.integers(0, 2600 if long_case else 700))
        hkv = int(rng.choice([1, 2, 4]))
        g = 1 if long_case else int(rng.choice([1, 2, 4]))
        d = 128 if long_case else int(rng.choice([64, 128]))
        causal = bool(rng.random() < 0.5)
        out = "f32" if rng.random() < 0.5 else "bf16"
        cases.append((b, nq, nk, hkv * g, hkv, d, causal, out))
    return cases


def _varlen_cases():
    rng = np.random.default_rng(20261203)
    cases = []
    for _ in range(6):
        n = int(rng.integers(1, 9))
        lq = [int(x) for x in rng.integers(0, 600, size=n)]
        lk = lq if rng.random() < 0.5 else [int(x) for x in rng.integers(0, 600, size=n)]
        hkv = int(rng.choice([1, 2]))
        g = int(rng.choice([1, 4]))
        d = int(rng.choice([64, 128]))
        cases.append((tuple(lq), tuple(lk), hkv * g, hkv, d, bool(rng.random() < 0.5)))
    return cases


def _variant_cases():
    rng = np.random.default_rng(20261204)
    cases = []
    for _ in range(8):
        b = int(rng.integers(1, 3))
        nq = int(rng.integers(1, 500))
        nk = nq if rng.random() < 0.6 else int(rng.integers(1, 500))
        hkv = int(rng.choice([1, 2]))
        g = int(rng.choice([1, 2, 4]))
        d = int(rng.choice([64, 128]))
        causal = bool(rng.random() < 0.5)
        window = tuple(int(x) if x >= 0 else -1 for x in rng.integers(-60, 300, size=2))
        cap = float(rng.choice([0.0, 0.0, 5.0, 30.0]))
        alibi = bool(rng.random() < 0.5)
        cases.append((b, nq, nk, hkv * g, hkv, d, causal, window, cap, alibi))
    return cases


def _decode_cases():
    rng = np.random.default_rng(20261205)
    cases = []
    for _ in range(6):
        b = int(rng.integers(1, 6))
        hkv = int(rng.choice([1, 2, 8]))
        g = int(rng.choice([1, 4, 8]))
        d = int(rng.choice([64, 128]))
        ncache = int(rng.integers(100, 3000))
        lens = tuple(int(x) for x in rng.integers(0, ncache + 1, size=b))
        chunk = int(rng.choice([0, 128, 384, 1024]))
        cases.append((b, hkv * g, hkv, ncache, lens, d, chunk))
    return cases


def _fp8_cases():
    rng = np.random.default_rng(20261206)
    cases = []
    for _ in range(5):
        b = int(rng.integers(1, 3))
        nq = int(rng.integers(1, 800))
        nk = nq if rng.random() < 0.6 else int(rng.integers(1, 800))
        hkv = int(rng.choice([1, 2]))
        g = int(rng.choice([1, 2, 4]))
        cases.append((b, nq, nk, hkv * g, hkv, bool(rng.random() < 0.5)))
    return cases


FIXED, VARLEN, VARIANT, DECODE, FP8 = (_fixed_cases(), _varlen_cases(), _variant_cases(),
                                       _decode_cases(), _fp8_cases())


@pytest.fixture(scope="module")
def fa():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_attention_84_amd as fa
    fa.load()
    return fa


@pytest.mark.parametrize("case", FIXED, ids=[str(c) for c in FIXED])
def test_random_fixed(fa, case):
    import torch
    bsz, nq, nk, hq, hkv, d, causal, out = case
    say("random fixed", case)
    q, k, v = W.make_fixed(bsz, hq, hkv, nq, nk, d, seed=1, wid=WID)
    scale = 1.0 / np.sqrt(d)
    o, lse = fa.attention(dev_bf16(q), dev_bf16(k), dev_bf16(v), causal=causal, scale=scale,
                          out_dtype=torch.float32 if out == "f32" else torch.bfloat16)
    torch.cuda.synchronize()
    orf, lrf = oracle.attention(q, k, v, scale, causal)
    check_o(host(o), orf, out == "bf16", str(case))
    check_lse(host(lse), lrf, str(case))


@pytest.mark.parametrize("case", VARLEN, ids=[str(c) for c in VARLEN])
def test_random_varlen(fa, case):
    import torch
    lq, lk, hq, hkv, d, causal = case
    say("random varlen", case)
    q, k, v, cu_q, cu_k = W.make_varlen(list(lq), list(lk), hq, hkv, d, seed=2, wid=WID)
    scale = 1.0 / np.sqrt(d)
    o, lse = fa.attention(dev_bf16(q), dev_bf16(k), dev_bf16(v), causal=causal, scale=scale,
                          cu_seqlens_q=dev_i32(cu_q), cu_seqlens_k=dev_i32(cu_k),
                          max_seqlen_q=max(lq), max_seqlen_k=max(lk), out_dtype=torch.float32)
    torch.cuda.synchronize()
    orf, lrf = oracle.attention_varlen(q, k, v, cu_q, cu_k, scale, causal)
    check_o(host(o), orf, False, str(case))
    check_lse(host(lse), lrf, str(case))


@pytest.mark.parametrize("case", VARIANT, ids=[str(c) for c in VARIANT])
def test_random_variants(fa, case):
    import torch
    bsz, nq, nk, hq, hkv, d, causal, window, cap, alibi = case
    say("random variants", case)
    q, k, v = W.make_fixed(bsz, hq, hkv, nq, nk, d, seed=3, wid=WID)
    sl = (2.0 ** (-8.0 * np.arange(1, hq + 1) / hq)).astype(np.float32) if alibi else None
    scale = 1.0 / np.sqrt(d)
    o, lse = fa.attention(dev_bf16(q), dev_bf16(k), dev_bf16(v), causal=causal, scale=scale,
                          window=window, softcap=cap,
                          alibi_slopes=None if sl is None else torch.from_numpy(sl).cuda(),
                          out_dtype=torch.float32)
    torch.cuda.synchronize()
    orf, lrf = V.attention_ext(q, k, v, scale, causal, window=window, softcap=cap, alibi=sl)
    check_o(host(o), orf, False, str(case))
    check_lse(host(lse), lrf, str(case))


@pytest.mark.parametrize("case", DECODE, ids=[str(c) for c in DECODE])
def test_random_decode(fa, case):
    import torch
    bsz, hq, hkv, ncache, lens, d, chunk = case
    say("random decode", case)
    lens = np.array(lens, np.int32)
    q, k, v = W.make_decode(bsz, hq, hkv, ncache, d, lens, seed=4, wid=WID, tail="nan")
    scale = 1.0 / np.sqrt(d)
    o, lse = fa.decode(dev_bf16(q), dev_bf16(k), dev_bf16(v), dev_i32(lens), scale=scale,
                       chunk=chunk, out_dtype=torch.float32)
    torch.cuda.synchronize()
    orf, lrf = oracle.decode(q, k, v, lens, scale)
    check_o(host(o), orf, False, str(case))
    check_lse(host(lse), lrf, str(case))


@pytest.mark.parametrize("case", FP8, ids=[str(c) for c in FP8])
def test_random_fp8(fa, case):
    import torch
    from test_gpu_fp8 import check, dev_u8
    bsz, nq, nk, hq, hkv, causal = case
    say("random fp8", case)
    q8, k8, v8, ds = W.make_fixed_fp8(bsz, hq, hkv, nq, nk, 128, seed=5, wid=WID)
    scale = 1 / np.sqrt(128)
    o, lse = fa.attention_fp8(dev_u8(q8), dev_u8(k8), dev_u8(v8), q_descale=ds[0],
                              k_descale=ds[1], v_descale=ds[2], causal=causal, scale=scale,
                              out_dtype=torch.float32)
    torch.cuda.synchronize()
    check(host(o), host(lse), q8, k8, v8, ds, scale, causal, False, str(case))
