"""The allocation-free KV-cache decode step (fa_fwd_decode_kvcache_noalloc)
against the entry point with a caller workspace (fa_fwd_decode_kvcache).

Both run the same kernels with the same split, so O, LSE and the updated
caches must agree bit for bit.  Two calls run back to back on the library's
scratch, the second on a smaller input, so the second starts from whatever the
first left there; a third call must match too after an over-size request was
refused.  The host-only tests check the refusal of requests larger than the
scratch, which happens before any device call.
"""
import os
import re

import numpy as np
import pytest

import workloads as W
from _gpu_helpers import dev_bf16, dev_i32, say
from exact_attention_84_amd import _lib

WID = 220
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x1000  # never dereferenced: the call is refused before any device work
WORKSPACE = 7


def noalloc(lib, **kw):
    a = dict(q=FAKE, kc=FAKE, vc=FAKE, kn=None, vn=None, lens=FAKE, table=None, mb=0, page=0,
             nblk=0, cos=None, sin=None, rdim=0, mpos=0, inter=0, o=FAKE, lse=FAKE, batch=64,
             hq=32, hkv=8, cap=32768, d=128, scale=0.088, chunk=0, odt=0, stream=None)
    a.update(kw)
    return lib.fa_fwd_decode_kvcache_noalloc(
        a["q"], a["kc"], a["vc"], a["kn"], a["vn"], a["lens"], a["table"], a["mb"], a["page"],
        a["nblk"], a["cos"], a["sin"], a["rdim"], a["mpos"], a["inter"], a["o"], a["lse"],
        a["batch"], a["hq"], a["hkv"], a["cap"], a["d"], a["scale"], a["chunk"], a["odt"],
        a["stream"])


def test_header_states_the_scratch_size():
    text = open(os.path.join(ROOT, "include", "fa.h")).read()
    m = re.search(r"#define FA_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", text)
    assert m, "FA_NOALLOC_SCRATCH_BYTES missing from fa.h"
    assert int(m.group(1)) << int(m.group(2)) == _lib.NOALLOC_SCRATCH_BYTES


@pytest.mark.parametrize("kw", [
    dict(hkv=1, chunk=128),                 # 64 x 32 rows x 256 splits x 129 floats = 270 MB
    dict(batch=256, hkv=8, cap=8192, d=64, chunk=128),  # 8192 rows x 64 splits x 65 floats
])
def test_noalloc_refuses_requests_beyond_the_scratch(kw):
    lib = _lib.load()
    # without rotary the call needs only the split partials
    need = lib.fa_decode_workspace_size(kw.get("batch", 64), kw.get("hq", 32),
                                        kw.get("cap", 32768), kw.get("d", 128), kw["chunk"])
    if need <= _lib.NOALLOC_SCRATCH_BYTES:
        pytest.skip(f"case needs only {need} bytes")
    assert noalloc(lib, **kw) == WORKSPACE
    msg = lib.fa_last_error().decode()
    assert "built-in scratch" in msg and str(need) in msg


def test_noalloc_accepts_the_decode_workload_size():
    # the split-KV decode workload (64 sequences, 32/8 heads, 32768 cache rows,
    # head_dim 128) with its built-in chunk and rotary fits in the scratch
    lib = _lib.load()
    chunk = 1536  # the built-in chunk for 64 x 8 (sequence, kv head) groups of 32768 keys
    need = lib.fa_decode_kvcache_workspace_size(64, 32, 32768, 128, chunk)
    assert 0 < need <= _lib.NOALLOC_SCRATCH_BYTES


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
    rng = np.random.default_rng(seed)
    c = dict(q=W.normal_bf16(seed, WID, 0, (b, hq, d)), lens=np.asarray(lens, np.int32),
             kn=W.normal_bf16(seed, WID, 1, (b, hkv, d)) if append else None,
             vn=W.normal_bf16(seed, WID, 2, (b, hkv, d)) if append else None, table=None)
    if page:
        nblk = cap // page
        pool = b * nblk + 2
        c["table"] = rng.permutation(pool)[: b * nblk].reshape(b, nblk).astype(np.int32)
        shape = (pool, page, hkv, d)
    else:
        shape = (b, cap, hkv, d)
    c["kc"] = W.normal_bf16(seed, WID, 3, shape)
    c["vc"] = W.normal_bf16(seed, WID, 4, shape)
    c["cos"], c["sin"] = tables(max(lens) + 2, rdim) if rdim else (None, None)
    return c


def run(fa, c, use_noalloc, out_dtype, chunk):
    """One step on fresh device copies of the caches; returns host results."""
    import torch
    t = lambda x: None if x is None else dev_bf16(x)
    f = lambda x: None if x is None else torch.from_numpy(x).cuda()
    q, kc, vc, kn, vn = t(c["q"]), t(c["kc"]), t(c["vc"]), t(c["kn"]), t(c["vn"])
    lens = dev_i32(c["lens"])
    table = None if c["table"] is None else dev_i32(c["table"])
    cos, sin = f(c["cos"]), f(c["sin"])
    out = torch.full(q.shape, float("nan"), dtype=out_dtype, device="cuda")
    lse = torch.full(q.shape[:2], float("nan"), dtype=torch.float32, device="cuda")
    kw = dict(k_new=kn, v_new=vn, block_table=table, rotary_cos=cos, rotary_sin=sin,
              chunk=chunk)
    torch.cuda.synchronize()
    if use_noalloc:
        before = torch.cuda.memory_stats().get("allocation.all.allocated", 0)
        fa.decode_kvcache_noalloc(q, kc, vc, lens, out, lse, **kw)
        after = torch.cuda.memory_stats().get("allocation.all.allocated", 0)
        assert after == before, "the allocation-free call allocated through torch"
    else:
        fa.decode_kvcache(q, kc, vc, lens, out=out, lse=lse, out_dtype=out_dtype, **kw)
    torch.cuda.synchronize()
    bits = lambda x: x.cpu().view(torch.int16).numpy().copy()
    return out.float().cpu().numpy(), lse.cpu().numpy(), bits(kc), bits(vc)


def same(a, b, what):
    for x, y, n in zip(a, b, ("O", "LSE", "key cache", "value cache")):
        assert x.shape == y.shape, f"{what}: {n} shape"
        assert np.array_equal(x, y, equal_nan=False), (
            f"{what}: {n} differs at {np.argwhere(x != y)[:3].tolist()}")
        if n in ("O", "LSE"):
            assert not np.isnan(x).any(), f"{what}: {n} left unwritten"


# (B, Hq, Hkv, d, capacity, lengths, page, append, rotary_dim, out dtype, chunk)
LARGE = (6, 32, 8, 128, 4096, [4095, 0, 1, 2000, 3333, 128], 256, True, 128, "f32", 0)
SMALL = (2, 8, 2, 128, 1024, [1000, 77], 0, False, 0, "bf16", 256)
SMALLEST = (3, 4, 4, 64, 512, [0, 129, 300], 128, True, 32, "f32", 128)


@pytest.mark.gpu
def test_noalloc_matches_workspace_entry_point_twice(fa):
    import torch
    dt = {"f32": torch.float32, "bf16": torch.bfloat16}
    for i, case in enumerate((LARGE, SMALL)):
        b, hq, hkv, d, cap, lens, page, append, rdim, odt, chunk = case
        say("noalloc call", i, case)
        c = make_case(b, hq, hkv, d, cap, lens, page, append, rdim, seed=i)
        got = run(fa, c, True, dt[odt], chunk)
        ref = run(fa, c, False, dt[odt], chunk)
        same(got, ref, f"call {i} {case}")


@pytest.mark.gpu
def test_noalloc_refusal_leaves_outputs_and_next_call_is_exact(fa):
    import torch
    q = torch.zeros(64, 32, 128, dtype=torch.bfloat16, device="cuda")
    lens = torch.zeros(64, dtype=torch.int32, device="cuda")
    cache = torch.zeros(64, 1, 1, 128, dtype=torch.bfloat16, device="cuda")
    out = torch.full((64, 32, 128), 7.0, dtype=torch.float32, device="cuda")
    lse = torch.full((64, 32), 7.0, dtype=torch.float32, device="cuda")
    # a request beyond the scratch is refused before the device is touched
    lib = fa.load()
    st = lib.fa_fwd_decode_kvcache_noalloc(
        q.data_ptr(), cache.data_ptr(), cache.data_ptr(), None, None, lens.data_ptr(), None, 0, 0,
        0, None, None, 0, 0, 0, out.data_ptr(), lse.data_ptr(), 64, 32, 1, 32768, 128, 0.088, 128,
        _lib.FA_DTYPE_F32, None)
    assert st == WORKSPACE
    torch.cuda.synchronize()
    assert (out == 7.0).all() and (lse == 7.0).all()
    say("noalloc after refusal", SMALLEST)
    b, hq, hkv, d, cap, lens_, page, append, rdim, odt, chunk = SMALLEST
    c = make_case(b, hq, hkv, d, cap, lens_, page, append, rdim, seed=5)
    same(run(fa, c, True, torch.float32, chunk), run(fa, c, False, torch.float32, chunk),
         f"after refusal {SMALLEST}")
