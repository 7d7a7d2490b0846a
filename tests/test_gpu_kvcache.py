"""Parity of the KV-cache decode step (fa_fwd_decode_kvcache: rotary, in-place
append, paged cache) with the fp64 oracle of oracle/kvcache.py, through the C
ABI (needs a GPU).

Bound: max-abs 1e-2 on O (fp32 output) and 1e-3 on LSE, as for the plain
decode.  The caches after the call are compared byte for byte, except the
appended key row under rotary: there each element may differ from the
oracle's by one bf16 ulp, because the kernel rotates in fp32 and the oracle in
fp64, and the two can fall on opposite sides of a bf16 rounding boundary.
"""
import numpy as np
import pytest

import oracle.kvcache as KV
import workloads as W
from _gpu_helpers import check_lse, check_o, dev_bf16, dev_i32, host, say

pytestmark = pytest.mark.gpu
WID = 210


@pytest.fixture(scope="module")
def fa():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_attention_84_amd as fa
    fa.load()
    return fa


def tables(max_pos, r, base=10000.0):
    inv = base ** (-np.arange(0, r, 2, dtype=np.float64) / r)
    ang = np.outer(np.arange(max_pos, dtype=np.float64), inv)
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


def make_case(b, hq, hkv, d, cap, lens, page, append, rdim, seed):
    """Inputs of one step as numpy arrays; paged when page > 0 (pages of the
    pool are handed out in a seeded random order)."""
    rng = np.random.default_rng(seed)
    q = W.normal_bf16(seed, WID, 0, (b, hq, d))
    kn = W.normal_bf16(seed, WID, 1, (b, hkv, d)) if append else None
    vn = W.normal_bf16(seed, WID, 2, (b, hkv, d)) if append else None
    if page:
        nblk = cap // page
        pool = b * nblk + 3                        # a few spare blocks
        table = rng.permutation(pool)[: b * nblk].reshape(b, nblk).astype(np.int32)
        kc = W.normal_bf16(seed, WID, 3, (pool, page, hkv, d))
        vc = W.normal_bf16(seed, WID, 4, (pool, page, hkv, d))
    else:
        table = None
        kc = W.normal_bf16(seed, WID, 3, (b, cap, hkv, d))
        vc = W.normal_bf16(seed, WID, 4, (b, cap, hkv, d))
    cos, sin = tables(max(lens) + 2, rdim) if rdim else (None, None)
    return dict(q=q, kn=kn, vn=vn, kc=kc, vc=vc, table=table, lens=np.asarray(lens, np.int32),
                cos=cos, sin=sin)


def run_gpu(fa, c, page, rdim, interleaved, scale, chunk=0):
    import torch
    t = lambda x: None if x is None else dev_bf16(x)
    kc, vc = dev_bf16(c["kc"]), dev_bf16(c["vc"])
    o, lse = fa.decode_kvcache(
        dev_bf16(c["q"]), kc, vc, dev_i32(c["lens"]), k_new=t(c["kn"]), v_new=t(c["vn"]),
        block_table=None if c["table"] is None else dev_i32(c["table"]),
        rotary_cos=None if not rdim else torch.from_numpy(c["cos"]).cuda(),
        rotary_sin=None if not rdim else torch.from_numpy(c["sin"]).cuda(),
        rotary_interleaved=interleaved, scale=scale, chunk=chunk, out_dtype=torch.float32)
    torch.cuda.synchronize()
    bits = lambda x: x.cpu().view(torch.int16).numpy().view(np.uint16)
    return host(o), host(lse), bits(kc), bits(vc)


def run_oracle(c, page, rdim, interleaved, scale):
    return KV.kvcache_step(c["q"], c["kc"], c["vc"], c["lens"], scale, k_new=c["kn"],
                           v_new=c["vn"], block_table=c["table"], page_size=page,
                           rotary_cos=c["cos"], rotary_sin=c["sin"], rotary_dim=rdim,
                           interleaved=interleaved)


def appended_rows(c, page):
    """Index tuples of the cache rows the step appends to."""
    if c["kn"] is None:
        return []
    return [KV.cache_row_index(b, int(t), c["table"], page) for b, t in enumerate(c["lens"])]


def check_caches(kg, vg, kr, vr, rows, rotary):
    """Caches equal byte for byte, except rotated appended key rows, whose
    elements may differ from the oracle's by one bf16 ulp."""
    kg, kr = kg.copy(), kr.copy()
    for idx in rows:
        if rotary:
            a = W.bf16_bits_to_f32(kg[idx]).astype(np.float64)
            b = W.bf16_bits_to_f32(kr[idx]).astype(np.float64)
            mag = np.maximum(np.abs(a), np.abs(b))
            ulp = np.exp2(np.floor(np.log2(np.maximum(mag, 1e-30))) - 7)
            assert (np.abs(a - b) <= ulp).all(), "appended key row"
        else:
            assert np.array_equal(kg[idx], kr[idx]), "appended key row"
        kg[idx] = kr[idx]
    assert np.array_equal(kg, kr), "key cache outside the appended rows"
    assert np.array_equal(vg, vr), "value cache"


CASES = [
    # (B, Hq, Hkv, d, capacity, lengths, page, append, rotary_dim, interleaved, chunk)
    (3, 8, 2, 128, 1024, [0, 255, 700], 256, False, 0, False, 0),      # paged decode only
    (3, 8, 2, 128, 1024, [1, 256, 1023], 128, True, 0, False, 256),    # paged append, page edges
    (2, 32, 8, 128, 768, [511, 767], 0, True, 0, False, 0),            # contiguous append
    (2, 8, 2, 128, 768, [100, 600], 0, True, 128, False, 0),           # rotary, rotate half
    (2, 8, 2, 128, 768, [100, 600], 256, True, 128, True, 0),          # rotary, interleaved, paged
    (3, 4, 4, 64, 512, [0, 129, 300], 128, True, 32, False, 128),      # d=64, partial rotary
    (2, 16, 1, 128, 512, [17, 400], 256, False, 64, False, 0),         # rotary of q only (no append)
]


@pytest.mark.parametrize("case", CASES, ids=[str(c) for c in CASES])
def test_kvcache_step_matches_oracle(fa, case):
    b, hq, hkv, d, cap, lens, page, append, rdim, inter, chunk = case
    say("kvcache", case)
    c = make_case(b, hq, hkv, d, cap, lens, page, append, rdim, seed=3)
    scale = 1.0 / np.sqrt(d)
    og, lg, kg, vg = run_gpu(fa, c, page, rdim, inter, scale, chunk)
    orf, lrf, kr, vr = run_oracle(c, page, rdim, inter, scale)
    check_o(og, orf, False, str(case))
    check_lse(lg, lrf, str(case))
    check_caches(kg, vg, kr, vr, appended_rows(c, page), rdim > 0)


def test_three_steps_in_a_row(fa):
    """Three decode steps, the host advancing cache_seqlens between them; the
    GPU cache carries over from step to step, the oracle's likewise."""
    import torch
    say("kvcache three steps")
    b, hq, hkv, d, cap, page, rdim = 2, 8, 2, 128, 512, 128, 128
    c = make_case(b, hq, hkv, d, cap, [126, 300], page, True, rdim, seed=5)
    cos, sin = tables(cap, rdim)
    kc_g, vc_g = dev_bf16(c["kc"]), dev_bf16(c["vc"])
    kc_o, vc_o = c["kc"], c["vc"]
    lens = c["lens"].copy()
    for step in range(3):
        q = W.normal_bf16(10 + step, WID, 0, (b, hq, d))
        kn = W.normal_bf16(10 + step, WID, 1, (b, hkv, d))
        vn = W.normal_bf16(10 + step, WID, 2, (b, hkv, d))
        o, lse = fa.decode_kvcache(dev_bf16(q), kc_g, vc_g, dev_i32(lens), k_new=dev_bf16(kn),
                                   v_new=dev_bf16(vn), block_table=dev_i32(c["table"]),
                                   rotary_cos=torch.from_numpy(cos).cuda(),
                                   rotary_sin=torch.from_numpy(sin).cuda(),
                                   out_dtype=torch.float32)
        torch.cuda.synchronize()
        orf, lrf, kc_o, vc_o = KV.kvcache_step(q, kc_o, vc_o, lens, 1 / np.sqrt(d), k_new=kn,
                                               v_new=vn, block_table=c["table"], page_size=page,
                                               rotary_cos=cos, rotary_sin=sin, rotary_dim=rdim)
        check_o(host(o), orf, False, f"step {step}")
        check_lse(host(lse), lrf, f"step {step}")
        lens = lens + 1
    # every byte of both caches after the three appends (the appended key
    # rows to one bf16 ulp)
    kg = kc_g.cpu().view(torch.int16).numpy().view(np.uint16)
    vg = vc_g.cpu().view(torch.int16).numpy().view(np.uint16)
    rows = [KV.cache_row_index(s, int(t), c["table"], page)
            for s in range(b) for t in range(int(c["lens"][s]), int(lens[s]))]
    check_caches(kg, vg, kc_o, vc_o, rows, True)


def test_plain_decode_entry_is_unchanged(fa):
    """fa_fwd_decode_splitkv routes through the same kernels with no append,
    no rotary and a contiguous cache: identical bytes to the KV-cache call."""
    import torch
    say("kvcache vs splitkv")
    c = make_case(2, 8, 2, 128, 1024, [300, 1024], 0, False, 0, seed=7)
    a = fa.decode(dev_bf16(c["q"]), dev_bf16(c["kc"]), dev_bf16(c["vc"]), dev_i32(c["lens"]),
                  out_dtype=torch.float32)
    bq = fa.decode_kvcache(dev_bf16(c["q"]), dev_bf16(c["kc"]), dev_bf16(c["vc"]),
                           dev_i32(c["lens"]), out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(a[0], bq[0]) and torch.equal(a[1], bq[1])


DEC = W.WORKLOADS[5]   # B=64, Hq=32, Hkv=8, cache 32768, d=128


def test_full_size_paged_append_rotary_sampled(fa):
    """The bench's paged KV-cache step at the decode workload's size (page
    256, shuffled block table, append and rotary), checked on sampled
    sequences that the oracle evaluates in full."""
    import torch
    say("kvcache full size")
    lens = W.workload_lengths(DEC, seed=0) - 1          # room for the appended token
    page, cap = 256, DEC.seqlen_k
    nblk = cap // page
    rng = np.random.default_rng(0)
    table = rng.permutation(DEC.batch * nblk).reshape(DEC.batch, nblk).astype(np.int32)
    kc = torch.empty((DEC.batch * nblk, page, DEC.heads_kv, DEC.head_dim), dtype=torch.bfloat16,
                     device="cuda").normal_()
    vc = torch.empty_like(kc).normal_()
    q = W.normal_bf16(0, WID, 0, (DEC.batch, DEC.heads_q, DEC.head_dim))
    kn = W.normal_bf16(0, WID, 1, (DEC.batch, DEC.heads_kv, DEC.head_dim))
    vn = W.normal_bf16(0, WID, 2, (DEC.batch, DEC.heads_kv, DEC.head_dim))
    cos, sin = tables(cap, DEC.head_dim)
    samples = (0, 31, 63)
    # the sampled sequences' blocks, taken before the call updates the pool;
    # the oracle sees them as a pool of their own with an identity table
    bits = lambda x: x.cpu().view(torch.int16).numpy().view(np.uint16)
    sub = {s: (bits(kc[torch.from_numpy(table[s]).long().cuda()]),
               bits(vc[torch.from_numpy(table[s]).long().cuda()])) for s in samples}
    o, lse = fa.decode_kvcache(dev_bf16(q), kc, vc, dev_i32(lens), k_new=dev_bf16(kn),
                               v_new=dev_bf16(vn), block_table=dev_i32(table),
                               rotary_cos=torch.from_numpy(cos).cuda(),
                               rotary_sin=torch.from_numpy(sin).cuda(), out_dtype=torch.float32)
    torch.cuda.synchronize()
    og, lg = host(o), host(lse)
    assert np.isfinite(og).all() and np.isfinite(lg).all()
    ident = np.arange(nblk, dtype=np.int32)[None, :]
    for s in samples:
        orf, lrf, _, _ = KV.kvcache_step(q[s:s + 1], sub[s][0], sub[s][1], lens[s:s + 1],
                                         DEC.scale, k_new=kn[s:s + 1], v_new=vn[s:s + 1],
                                         block_table=ident, page_size=page,
                                         rotary_cos=cos, rotary_sin=sin,
                                         rotary_dim=DEC.head_dim)
        check_o(og[s:s + 1], orf, False, f"seq {s}")
        check_lse(lg[s:s + 1], lrf, f"seq {s}")
