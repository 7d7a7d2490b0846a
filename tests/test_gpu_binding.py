"""The Python binding's own checks and stream handling (needs a GPU for device
tensors; the rejected calls never reach a kernel)."""
import numpy as np
import pytest

import oracle
import workloads as W
from _gpu_helpers import check_lse, check_o, dev_bf16, dev_i32, host, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_attention_84_amd as fa
    fa.load()
    return fa


def test_caller_outputs_are_checked(fa):
    import torch
    say("binding: caller-provided outputs")
    lens = np.array([300, 77], np.int32)
    q, kc, vc = W.make_decode(2, 8, 2, 512, 128, lens, seed=3, wid=301)
    qd, kd, vd, ld = dev_bf16(q), dev_bf16(kc), dev_bf16(vc), dev_i32(lens)
    with pytest.raises(ValueError):
        fa.decode(qd, kd, vd, ld, out=torch.empty((2, 4, 128), dtype=torch.bfloat16, device="cuda"))
    with pytest.raises(ValueError):
        fa.decode(qd, kd, vd, ld, lse=torch.empty((2, 4), dtype=torch.float32, device="cuda"))
    with pytest.raises(ValueError):
        fa.decode_kvcache(qd, kd, vd, ld,
                          out=torch.empty((2, 8, 64), dtype=torch.bfloat16, device="cuda"))
    with pytest.raises(ValueError):
        fa.decode_kvcache(qd, kd, vd, ld, lse=torch.empty((3, 8), dtype=torch.float32,
                                                           device="cuda"))
    op = torch.zeros((16, 3, 128), dtype=torch.float32, device="cuda")
    lp = torch.zeros((16, 3), dtype=torch.float32, device="cuda")
    with pytest.raises(TypeError):  # out dtype differs from out_dtype (fp32 by default)
        fa.combine(op, lp, out=torch.empty((16, 128), dtype=torch.bfloat16, device="cuda"))
    with pytest.raises(ValueError):
        fa.combine(op, lp, out=torch.empty((8, 128), dtype=torch.float32, device="cuda"))
    with pytest.raises(ValueError):
        fa.combine(op, lp, lse=torch.empty((15,), dtype=torch.float32, device="cuda"))


def test_side_stream_calls_match_the_oracle(fa):
    """Decode and the backward on a stream other than the current one, with
    every workspace and output allocated by the binding, while the current
    stream allocates and fills memory of the same sizes: results must equal
    those of the same calls on the current stream (the library is bitwise
    deterministic) and match the oracle."""
    import torch
    say("binding: side stream")
    side = torch.cuda.Stream()
    lens = np.array([1500, 999, 2048], np.int32)
    q, kc, vc = W.make_decode(3, 8, 2, 2048, 128, lens, seed=4, wid=302, tail="nan")
    qd, kd, vd, ld = dev_bf16(q), dev_bf16(kc), dev_bf16(vc), dev_i32(lens)
    o_ref, l_ref = fa.decode(qd, kd, vd, ld, chunk=256, out_dtype=torch.float32)
    torch.cuda.synchronize()
    results = []
    for _ in range(3):
        o, l = fa.decode(qd, kd, vd, ld, chunk=256, out_dtype=torch.float32, stream=side)
        # memory of the same sizes, written on the current stream meanwhile
        junk = [torch.full((n,), float("nan"), device="cuda") for n in (o.numel(), 4 << 20)]
        results.append((o, l, junk))
    side.synchronize()
    torch.cuda.synchronize()
    for o, l, _ in results:
        assert torch.equal(o, o_ref) and torch.equal(l, l_ref)
    orf, lrf = oracle.decode(q, kc, vc, lens, 1.0 / np.sqrt(128))
    check_o(host(o_ref), orf, False, "side-stream decode")
    check_lse(host(l_ref), lrf, "side-stream decode")

    qf, kf, vf = W.make_fixed(2, 4, 2, 300, 300, 128, seed=5, wid=303)
    do = W.make_dout(qf.shape, seed=5, wid=303)
    qd, kd, vd, dod = dev_bf16(qf), dev_bf16(kf), dev_bf16(vf), dev_bf16(do)
    ob, lb = fa.attention(qd, kd, vd, causal=True)
    ref = fa.attention_backward(qd, kd, vd, ob, lb, dod, causal=True)
    torch.cuda.synchronize()
    got = fa.attention_backward(qd, kd, vd, ob, lb, dod, causal=True, stream=side)
    junk = [torch.full((t.numel(),), float("nan"), device="cuda") for t in got]
    side.synchronize()
    torch.cuda.synchronize()
    for a, b in zip(got, ref):
        assert torch.equal(a, b)
    del junk
