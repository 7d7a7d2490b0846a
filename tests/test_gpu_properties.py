"""Properties of the HIP path that hold at any size (needs a GPU).

Closed forms at full workload shapes (equal scores give prefix means and
LSE = ln(i+1); constant V gives O = V), run-to-run bitwise determinism,
isolation of packed sequences, and independence of the split count in the
decode path.
"""
import math

import numpy as np
import pytest

import workloads as W
from _gpu_helpers import LSE_TOL, O_TOL, dev_bf16, dev_i32, host, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_attention_84_amd as fa
    fa.load()
    return fa


@pytest.mark.parametrize("wid", [2, 3])
def test_equal_scores_give_prefix_means(fa, wid):
    """Q = 0 at the full workload shape: causal row i is the mean of V[0..i]
    and LSE_i = ln(i + 1)."""
    import torch
    w = W.WORKLOADS[wid]
    say("prefix means", w.name)
    inp = W.make_workload(w, seed=1)
    q = torch.zeros((w.batch, w.seqlen_q, w.heads_q, w.head_dim), dtype=torch.bfloat16,
                    device="cuda")
    v = dev_bf16(inp["v"])
    o, lse = fa.attention(q, dev_bf16(inp["k"]), v, causal=True, scale=w.scale,
                          out_dtype=torch.float32)
    g = w.heads_q // w.heads_kv
    vf = v.float()
    ref = torch.cumsum(vf, dim=1) / torch.arange(1, w.seqlen_q + 1, device="cuda").view(
        1, -1, 1, 1)
    ref = ref.repeat_interleave(g, dim=2)
    err_o = (o - ref).abs().max().item()
    lref = torch.log(torch.arange(1, w.seqlen_q + 1, device="cuda", dtype=torch.float64))
    err_l = (lse.double() - lref.view(1, -1, 1)).abs().max().item()
    say("err", err_o, err_l)
    assert err_o <= O_TOL and err_l <= LSE_TOL


def test_constant_v_gives_constant_o(fa):
    """O = c exactly in the definition; the kernel multiplies bf16-rounded
    probabilities with V but divides by the fp32 sum, so it is off by at most
    2^-9 |c| (the relative rounding bound of bf16) from c."""
    import torch
    w = W.WORKLOADS[2]
    say("constant V")
    inp = W.make_workload(w, seed=2)
    v = torch.full((w.batch, w.seqlen_k, w.heads_kv, w.head_dim), -2.5, dtype=torch.bfloat16,
                   device="cuda")
    for causal in (False, True):
        o, _ = fa.attention(dev_bf16(inp["q"]), dev_bf16(inp["k"]), v, causal=causal,
                            scale=w.scale, out_dtype=torch.float32)
        assert (o + 2.5).abs().max().item() <= 2.5 * 2.0 ** -9


def test_causal_row_zero_is_v0(fa):
    import torch
    w = W.WORKLOADS[3]
    say("row 0")
    inp = W.make_workload(w, seed=3)
    qd, kd, vd = dev_bf16(inp["q"]), dev_bf16(inp["k"]), dev_bf16(inp["v"])
    o, lse = fa.attention(qd, kd, vd, causal=True, scale=w.scale, out_dtype=torch.float32)
    g = w.heads_q // w.heads_kv
    v0 = vd[:, 0].float().repeat_interleave(g, dim=1)
    assert (o[:, 0] - v0).abs().max().item() <= 1e-6
    s00 = (qd[:, 0].double() * kd[:, 0].double().repeat_interleave(g, dim=1)).sum(-1) * w.scale
    assert (lse[:, 0].double() - s00).abs().max().item() <= LSE_TOL


def test_bitwise_deterministic(fa):
    import torch
    w = W.WORKLOADS[2]
    say("determinism")
    inp = W.make_workload(w, seed=4)
    args = [dev_bf16(inp[x]) for x in "qkv"]
    o1, l1 = fa.attention(*args, causal=True, scale=w.scale)
    o2, l2 = fa.attention(*args, causal=True, scale=w.scale)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_varlen_sequences_are_isolated(fa):
    """Changing sequence s+1 leaves sequence s bitwise unchanged, and each
    packed sequence equals its own fixed-length call."""
    import torch
    lens = [300, 129, 1, 64, 513]
    say("varlen isolation")
    q, k, v, cu, _ = W.make_varlen(lens, lens, 8, 2, 128, seed=5, wid=104)
    qd, kd, vd = dev_bf16(q), dev_bf16(k), dev_bf16(v)
    cud = dev_i32(cu)
    o1, l1 = fa.attention(qd, kd, vd, causal=True, cu_seqlens_q=cud, max_seqlen_q=max(lens),
                          max_seqlen_k=max(lens), out_dtype=torch.float32)
    k2, v2 = kd.clone(), vd.clone()
    k2[cu[1]:cu[2]] = -k2[cu[1]:cu[2]]
    v2[cu[1]:cu[2]] = 3 * v2[cu[1]:cu[2]]
    o2, l2 = fa.attention(qd, k2, v2, causal=True, cu_seqlens_q=cud, max_seqlen_q=max(lens),
                          max_seqlen_k=max(lens), out_dtype=torch.float32)
    torch.cuda.synchronize()
    keep = torch.ones(q.shape[0], dtype=torch.bool, device="cuda")
    keep[cu[1]:cu[2]] = False
    assert torch.equal(o1[keep], o2[keep]) and torch.equal(l1[keep], l2[keep])
    for s in range(len(lens)):
        a, b = int(cu[s]), int(cu[s + 1])
        of, lf = fa.attention(qd[a:b][None].contiguous(), kd[a:b][None].contiguous(),
                              vd[a:b][None].contiguous(), causal=True, out_dtype=torch.float32)
        assert torch.equal(of[0], o1[a:b]) and torch.equal(lf[0], l1[a:b])


def test_decode_split_count_invariance(fa):
    import torch
    say("split invariance")
    lens = np.array([4000, 1, 2500, 3333], np.int32)
    q, k, v = W.make_decode(4, 32, 8, 4096, 128, lens, seed=6, wid=105, tail="nan")
    args = [dev_bf16(q), dev_bf16(k), dev_bf16(v), dev_i32(lens)]
    outs = [fa.decode(*args, chunk=c, out_dtype=torch.float32) for c in (128, 384, 1024, 4096, 0)]
    torch.cuda.synchronize()
    o0, l0 = outs[-2]  # 4096: one split per sequence
    for o, l in outs:
        assert (o - o0).abs().max().item() <= 2e-3
        assert (l - l0).abs().max().item() <= 2e-4


def test_decode_matches_prefill_with_one_query(fa):
    """A decode call equals the prefill path with Lq = 1 and bottom-right
    causal masking over the valid cache prefix."""
    import torch
    say("decode vs prefill")
    lens = np.array([777, 2048], np.int32)
    q, k, v = W.make_decode(2, 8, 2, 2048, 128, lens, seed=7, wid=106)
    od, ld = fa.decode(dev_bf16(q), dev_bf16(k), dev_bf16(v), dev_i32(lens),
                       out_dtype=torch.float32)
    for b in range(2):
        n = int(lens[b])
        op, lp = fa.attention(dev_bf16(q[b][None, None]), dev_bf16(k[b:b + 1, :n]),
                              dev_bf16(v[b:b + 1, :n]), causal=True, out_dtype=torch.float32)
        assert (op[0, 0] - od[b]).abs().max().item() <= 2e-3
        assert (lp[0, 0] - ld[b]).abs().max().item() <= 2e-4


def test_one_hot_v_returns_the_probabilities(fa):
    """V = I (as many keys as head dims) makes O the probability matrix
    itself: entries >= 0, each row summing to 1, equal to the definition's
    softmax.  P is rounded to bf16 before the product while l sums the fp32
    values, so a row sums to 1 within the bf16 relative rounding 2^-9."""
    import torch
    import oracle
    d, nk = 128, 128
    say("one-hot V")
    q, k, _ = W.make_fixed(2, 4, 2, nk, nk, d, seed=8, wid=107)  # every row sees a key
    eye = np.broadcast_to(np.eye(nk, d, dtype=np.float32), (2, 2, nk, d)).transpose(0, 2, 1, 3)
    v = W.round_f32_to_bf16_bits(np.ascontiguousarray(eye))
    for causal in (False, True):
        o, lse = fa.attention(dev_bf16(q), dev_bf16(k), dev_bf16(v), causal=causal,
                              out_dtype=torch.float32)
        o = host(o)
        assert o.min() >= -1e-6
        assert np.abs(o.sum(-1) - 1.0).max() <= 2.0 ** -9
        orf, lrf = oracle.attention(q, k, v, 1.0 / np.sqrt(d), causal)
        assert np.abs(o - orf).max() <= O_TOL
        assert np.abs(host(lse) - lrf).max() <= LSE_TOL


def plain_bf16_attention(q, k, v, scale, causal):
    """Unfused attention as eager PyTorch computes it on bf16 tensors (on the
    CPU): S = Q K^T stored as bf16, scaled in bf16, softmax in fp32 stored as
    bf16, O = P V stored as bf16.  Lq = Lk."""
    import torch
    tq, tk, tv = (torch.from_numpy(W.bf16_bits_to_f32(x)).to(torch.bfloat16).transpose(1, 2)
                  .contiguous() for x in (q, k, v))
    s = torch.matmul(tq, tk.transpose(-1, -2).contiguous())
    s = s * torch.tensor(scale, dtype=torch.bfloat16)
    if causal:
        n = s.shape[-1]
        s = s.masked_fill(~torch.ones(n, n, dtype=torch.bool).tril(), float("-inf"))
    p = torch.softmax(s.float(), dim=-1).to(torch.bfloat16)
    return torch.matmul(p, tv).transpose(1, 2).float().numpy().astype(np.float64)


def test_error_within_twice_a_plain_bf16_attention(fa):
    """Diagnostic error budget: against the fp64 definition, the fused
    kernel's bf16 output is no worse than twice the error of plain unfused
    bf16 attention."""
    import oracle
    say("error budget vs plain bf16")
    bsz, n, h, d = 1, 1024, 4, 128
    scale = 1.0 / np.sqrt(d)
    q, k, v = W.make_fixed(bsz, h, h, n, n, d, seed=9, wid=108)
    for causal in (False, True):
        og, _ = fa.attention(dev_bf16(q), dev_bf16(k), dev_bf16(v), causal=causal, scale=scale)
        ref, _ = oracle.attention(q, k, v, scale, causal)
        err_gpu = np.abs(host(og) - ref).max()
        err_plain = np.abs(plain_bf16_attention(q, k, v, scale, causal) - ref).max()
        say("causal", causal, "fused", err_gpu, "plain bf16", err_plain)
        assert err_gpu <= 2.0 * err_plain


@pytest.mark.parametrize("case", [(1100, False), (1100, True), (2048, True)],
                         ids=["n1100", "n1100-causal", "n2048-causal-8waves"])
def test_rising_scores_move_the_reference(fa, case):
    """Scores that grow along the keys (by about 2 log2 units per 64-key
    tile) make every row's running maximum pass its reference again and
    again inside the pipelined key loop, so the probabilities of many steps
    are taken against a reference that must move: the result still matches
    the oracle."""
    import torch
    import oracle
    from _gpu_helpers import check_lse, check_o
    n, causal = case
    say("rising scores", case)
    q, k, v = W.make_rising(1, 4, 2, n, 128, seed=3, wid=240)
    scale = 1 / math.sqrt(128)
    o, lse = fa.attention(dev_bf16(q), dev_bf16(k), dev_bf16(v), causal=causal, scale=scale,
                          out_dtype=torch.float32)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention(q, k, v, scale, causal)
    say("err", check_o(host(o), o_ref, False, str(case)), check_lse(host(lse), l_ref, str(case)))
