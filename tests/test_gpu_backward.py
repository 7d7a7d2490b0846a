"""Parity of the HIP backward (dQ, dK, dV) with the fp64 gradient oracle,
through the C ABI (needs a GPU).

The backward takes O and the logsumexp as inputs.  The parity cases feed it
the oracle's own forward (O rounded to bf16, LSE to fp32), so what is tested
is the backward alone; one case chains the HIP forward into the HIP backward.
The per-element tolerance is derived from the kernels' arithmetic in
``_grad_bounds``.
"""
import numpy as np
import pytest

import oracle
import workloads as W
from _gpu_helpers import dev_bf16, dev_i32, host, say
from _grad_bounds import (bf16_bits_of, check_grad, fixed_bounds, oracle_forward_inputs,
                          varlen_bounds)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_attention_84_amd as fa
    fa.load()
    return fa


def run_bwd(fa, q, k, v, o_bits, lse32, do, causal, scale, grad_dtype, **kw):
    import torch
    dq, dk, dv = fa.attention_backward(dev_bf16(q), dev_bf16(k), dev_bf16(v), dev_bf16(o_bits),
                                       torch.from_numpy(lse32).cuda(), dev_bf16(do),
                                       causal=causal, scale=scale, grad_dtype=grad_dtype, **kw)
    torch.cuda.synchronize()
    return host(dq), host(dk), host(dv)


FIXED_CASES = [
    # (B, Nq, Nk, Hq, Hkv, d, causal)
    (2, 300, 300, 4, 2, 128, False),
    (2, 300, 300, 4, 2, 128, True),
    (1, 257, 257, 2, 2, 64, False),
    (1, 257, 257, 2, 2, 64, True),
    (2, 100, 333, 4, 1, 128, True),   # fewer queries than keys (bottom-right)
    (1, 333, 100, 4, 4, 128, True),   # more queries than keys: early rows see nothing
    (1, 1, 1, 1, 1, 128, True),
    (3, 17, 17, 2, 1, 64, True),
    (1, 64, 700, 2, 2, 128, False),
    (2, 200, 0, 2, 2, 64, False),     # no keys: dQ = 0
    (2, 0, 50, 2, 1, 128, False),     # no queries: dK = dV = 0
    (3, 200, 200, 6, 3, 128, True),   # 9 (sequence, kv-head) groups
    (1, 520, 520, 8, 1, 128, True),   # MQA: 8 query heads summed into one
]


@pytest.mark.parametrize("case", FIXED_CASES, ids=[str(c) for c in FIXED_CASES])
@pytest.mark.parametrize("gdt", ["f32", "bf16"])
def test_fixed_backward_matches_oracle(fa, case, gdt):
    import torch
    bsz, nq, nk, hq, hkv, d, causal = case
    say("bwd fixed", case, gdt)
    q, k, v = W.make_fixed(bsz, hq, hkv, nq, nk, d, seed=11, wid=201, k_mult=1.5)
    do = W.make_dout(q.shape, seed=11, wid=201)
    scale = 1.0 / np.sqrt(d)
    o_bits, lse32, o_in, lse_in = oracle_forward_inputs(q, k, v, scale, causal)
    got = run_bwd(fa, q, k, v, o_bits, lse32, do, causal, scale,
                  torch.float32 if gdt == "f32" else torch.bfloat16)
    ref = oracle.attention_grad(q, k, v, do, scale, causal)
    bnd = fixed_bounds(q, k, v, do, o_in, lse_in, scale, causal)
    for name, g, r, b in zip(("dQ", "dK", "dV"), got, ref, bnd):
        check_grad(name, g, r, b, gdt == "bf16", str(case))


VARLEN_CASES = [
    ([1, 17, 300, 0, 129, 64, 65], None, 4, 2, 128),
    ([5, 250, 3, 77], [9, 300, 1, 77], 8, 2, 128),   # separate key lengths
    ([130, 1, 64], None, 2, 1, 64),
    ([300, 1, 513, 128, 129, 0, 257, 64, 700, 33], None, 4, 2, 128),
]


@pytest.mark.parametrize("case", VARLEN_CASES, ids=[str(c[0]) for c in VARLEN_CASES])
@pytest.mark.parametrize("causal", [False, True])
def test_varlen_backward_matches_oracle(fa, case, causal):
    import torch
    lq, lk, hq, hkv, d = case
    lk = lq if lk is None else lk
    say("bwd varlen", case, causal)
    q, k, v, cu_q, cu_k = W.make_varlen(lq, lk, hq, hkv, d, seed=12, wid=202)
    do = W.make_dout(q.shape, seed=12, wid=202, cu_q=cu_q)
    scale = 1.0 / np.sqrt(d)
    o_bits, lse32, o_in, lse_in = oracle_forward_inputs(q, k, v, scale, causal, cu_q, cu_k)
    got = run_bwd(fa, q, k, v, o_bits, lse32, do, causal, scale, torch.float32,
                  cu_seqlens_q=dev_i32(cu_q), cu_seqlens_k=dev_i32(cu_k),
                  max_seqlen_q=max(lq), max_seqlen_k=max(lk))
    ref = oracle.attention_grad_varlen(q, k, v, do, cu_q, cu_k, scale, causal)
    bnd = varlen_bounds(q, k, v, do, o_in, lse_in, cu_q, cu_k, scale, causal)
    for name, g, r, b in zip(("dQ", "dK", "dV"), got, ref, bnd):
        check_grad(name, g, r, b, False, str(case))


def test_backward_is_deterministic(fa):
    """No atomics: two calls give bitwise identical gradients."""
    import torch
    say("bwd determinism")
    q, k, v = W.make_fixed(2, 8, 2, 700, 700, 128, seed=13, wid=203)
    do = W.make_dout(q.shape, seed=13, wid=203)
    o, lse = oracle.attention(q, k, v, 1 / np.sqrt(128), True)
    args = (dev_bf16(q), dev_bf16(k), dev_bf16(v), dev_bf16(bf16_bits_of(o)),
            torch.from_numpy(lse.astype(np.float32)).cuda(), dev_bf16(do))
    a = fa.attention_backward(*args, causal=True)
    b = fa.attention_backward(*args, causal=True)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_caller_workspace_matches_own(fa):
    import torch
    say("bwd workspace")
    q, k, v = W.make_fixed(1, 4, 2, 130, 130, 64, seed=14, wid=204)
    do = W.make_dout(q.shape, seed=14, wid=204)
    o, lse = oracle.attention(q, k, v, 0.125, False)
    args = (dev_bf16(q), dev_bf16(k), dev_bf16(v), dev_bf16(bf16_bits_of(o)),
            torch.from_numpy(lse.astype(np.float32)).cuda(), dev_bf16(do))
    ws = torch.full((fa.bwd_workspace_size(1, 4, 130) + 256,), 0x7F, dtype=torch.uint8,
                    device="cuda")
    a = fa.attention_backward(*args, workspace=ws)
    b = fa.attention_backward(*args)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_forward_then_backward_matches_oracle(fa):
    """The HIP forward's O (bf16) and LSE feed the HIP backward; the bound
    takes their measured deviation from the exact forward."""
    import torch
    say("bwd after hip forward")
    case = (2, 300, 300, 4, 2, 128, True)
    bsz, nq, nk, hq, hkv, d, causal = case
    q, k, v = W.make_fixed(bsz, hq, hkv, nq, nk, d, seed=15, wid=205, k_mult=1.5)
    do = W.make_dout(q.shape, seed=15, wid=205)
    scale = 1.0 / np.sqrt(d)
    qd, kd, vd = dev_bf16(q), dev_bf16(k), dev_bf16(v)
    o, lse = fa.attention(qd, kd, vd, causal=causal, scale=scale, out_dtype=torch.bfloat16)
    dq, dk, dv = fa.attention_backward(qd, kd, vd, o, lse, dev_bf16(do), causal=causal,
                                       scale=scale)
    torch.cuda.synchronize()
    ref = oracle.attention_grad(q, k, v, do, scale, causal)
    bnd = fixed_bounds(q, k, v, do, host(o), host(lse), scale, causal)
    for name, g, r, b in zip(("dQ", "dK", "dV"), (host(dq), host(dk), host(dv)), ref, bnd):
        check_grad(name, g, r, b, False, str(case))


FULL = W.WORKLOADS[2]   # batched MHA B=4, H=16, N=2048, d=128


@pytest.mark.parametrize("causal", [False, True])
def test_full_size_backward_sampled_heads(fa, causal):
    """The bench's backward launch (B=4, H=16, N=2048, d=128), checked in
    full on sampled (sequence, head) pairs; each head's gradients depend on
    that head alone."""
    import torch
    say("bwd full", FULL.name, causal)
    inp = W.make_workload(FULL)
    q, k, v = inp["q"], inp["k"], inp["v"]
    do = W.make_dout(q.shape, seed=0, wid=FULL.wid)
    scale = FULL.scale
    qd, kd, vd = dev_bf16(q), dev_bf16(k), dev_bf16(v)
    o, lse = fa.attention(qd, kd, vd, causal=causal, scale=scale, out_dtype=torch.bfloat16)
    dq, dk, dv = fa.attention_backward(qd, kd, vd, o, lse, dev_bf16(do), causal=causal,
                                       scale=scale)
    torch.cuda.synchronize()
    for g in (dq, dk, dv):
        assert torch.isfinite(g).all()
    o_h, lse_h = host(o), host(lse)
    for b, h in ((0, 0), (1, 7), (3, 15)):
        sl = (slice(b, b + 1), slice(None), slice(h, h + 1))
        qs, ks, vs, ds_ = q[sl], k[sl], v[sl], do[sl]
        ref = oracle.attention_grad(qs, ks, vs, ds_, scale, causal)
        bnd = fixed_bounds(qs, ks, vs, ds_, o_h[sl], lse_h[sl], scale, causal)
        for name, gt, r, bb in zip(("dQ", "dK", "dV"), (dq, dk, dv), ref, bnd):
            check_grad(name, host(gt[b:b + 1, :, h:h + 1]), r, bb, False, f"({b},{h})")
