"""Parity of the FP8 forward (fa_fwd_fp8) with the fp64 oracle of
oracle/fp8.py, through the C ABI (needs a GPU).

The result is exact attention of the descaled E4M3 inputs.  The kernel's
error has three sources, each bounded here:
  * the probabilities rounded to E4M3 before the P V product:
    oracle.fp8.p_rounding_bound, elementwise on O;
  * the FP8 matrix core's accumulation of the 64-term score sums, which is
    not exact fp32 (measured on gfx950: errors up to about 2^-12 of the
    largest product of a sum; taken as 2^-11 per 64-term sum, two sums per
    score): |ds_i| <= 2^-10 scale dq dk max_k |q8_ik| max_jk |k8_jk|, which
    moves the LSE by at most ds_i and O by at most 4 ds_i max |v|;
  * fp32 arithmetic elsewhere: 2e-3 on O, 1e-3 on the LSE (the bf16 path's
    LSE bound), plus half a bf16 ulp for a bf16 O.
The worst-case bound on the rounding of P is loose, so the RMS of the O error
over a case with many elements is also held to 1.5 times the RMS error of the
oracle's reference rounding (attention_fp8_rounded_p): a misplaced or dropped
key, well inside the worst-case bound, fails that."""
import numpy as np
import pytest

import oracle.fp8 as F
import workloads as W
from _gpu_helpers import bf16_half_ulp, dev_i32, host, say

pytestmark = pytest.mark.gpu
WID = 230
LSE_TOL = 1e-3
O_SLACK = 2e-3


@pytest.fixture(scope="module")
def fa():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_attention_84_amd as fa
    fa.load()
    return fa


def dev_u8(x):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.uint8)).cuda()


def score_err(q8, k8, ds, scale):
    """Per query row bound on the score error of the FP8 matrix core, shape
    q8.shape[:-1] (max over the whole K tensor, which covers every key)."""
    qmax = np.abs(F.e4m3_to_f64(q8)).max(axis=-1)
    kmax = np.abs(F.e4m3_to_f64(k8)).max()
    return 2.0 ** -10 * scale * ds[0] * ds[1] * qmax * kmax


def check(o_gpu, lse_gpu, q8, k8, v8, ds, scale, causal, bf16_out, what, rms=True):
    """Compare one fixed-length batch (B, N, H, d) with the oracle."""
    o_ex, l_ex = F.attention_fp8(q8, k8, v8, *ds, scale=scale, causal=causal)
    bound = F.p_rounding_bound(q8, k8, v8, *ds, scale=scale, causal=causal)
    dsc = score_err(q8, k8, ds, scale)
    vmax = np.abs(F.dequantize(v8, ds[2])).max()
    tol = bound + (4 * dsc * vmax)[..., None] + O_SLACK
    if bf16_out:
        tol = tol + bf16_half_ulp(o_ex)
    assert np.isfinite(o_gpu).all(), f"{what}: non-finite O"
    err = np.abs(o_gpu - o_ex)
    bad = err > tol
    assert not bad.any(), (f"{what}: O error {err.max():.3e} over its bound at "
                           f"{np.argwhere(bad)[:3].tolist()}")
    fin = np.isfinite(l_ex)
    assert np.array_equal(np.isneginf(lse_gpu), np.isneginf(l_ex)), f"{what}: LSE -inf rows"
    lerr = np.abs(lse_gpu[fin] - l_ex[fin])
    assert (lerr <= LSE_TOL + dsc[fin]).all(), f"{what}: LSE error {lerr.max(initial=0):.3e}"
    if rms and err.size >= 20000:
        ref = F.attention_fp8_rounded_p(q8, k8, v8, *ds, scale=scale, causal=causal)
        r_gpu = np.sqrt(np.mean(err ** 2))
        r_ref = np.sqrt(np.mean((ref - o_ex) ** 2))
        assert r_gpu <= 1.5 * r_ref + 1e-4, f"{what}: O RMS error {r_gpu:.3e} vs {r_ref:.3e}"
    return float(err.max())


CASES = [
    # (B, Nq, Nk, Hq, Hkv, causal)
    (2, 300, 300, 4, 2, False),
    (2, 300, 300, 4, 2, True),
    (1, 257, 400, 2, 2, True),       # Lq < Lk
    (1, 400, 257, 2, 1, True),       # Lq > Lk: the first 143 rows see no key
    (3, 64, 64, 2, 2, False),        # one exact tile
    (1, 1, 1000, 4, 4, False),       # one query
    (2, 1100, 1100, 4, 2, True),     # several causal tile pairs
    (1, 2048, 2048, 2, 1, True),     # 8-wave workgroups
    (1, 2048, 1500, 2, 2, False),
]


@pytest.mark.parametrize("case", CASES, ids=[str(c) for c in CASES])
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_fp8_matches_oracle(fa, case, out):
    import torch
    bsz, nq, nk, hq, hkv, causal = case
    say("fp8", case, out)
    q8, k8, v8, ds = W.make_fixed_fp8(bsz, hq, hkv, nq, nk, 128, seed=31, wid=WID)
    scale = 1 / np.sqrt(128)
    o, lse = fa.attention_fp8(dev_u8(q8), dev_u8(k8), dev_u8(v8), q_descale=ds[0],
                              k_descale=ds[1], v_descale=ds[2], causal=causal, scale=scale,
                              out_dtype=torch.float32 if out == "f32" else torch.bfloat16)
    torch.cuda.synchronize()
    check(host(o), host(lse), q8, k8, v8, ds, scale, causal, out == "bf16", str(case))


def test_fp8_accepts_float8_tensors_and_other_descales(fa):
    import torch
    say("fp8 float8 dtype")
    q8, k8, v8, _ = W.make_fixed_fp8(1, 2, 1, 200, 300, 128, seed=32, wid=WID)
    ds = (0.01, 0.02, 0.5)
    as_f8 = lambda x: dev_u8(x).view(torch.float8_e4m3fn)  # noqa: E731
    o, lse = fa.attention_fp8(as_f8(q8), as_f8(k8), as_f8(v8), q_descale=ds[0], k_descale=ds[1],
                              v_descale=ds[2], causal=False, scale=0.3, out_dtype=torch.float32)
    torch.cuda.synchronize()
    check(host(o), host(lse), q8, k8, v8, ds, 0.3, False, False, "float8 dtype")


@pytest.mark.parametrize("causal", [False, True])
def test_fp8_varlen_matches_oracle(fa, causal):
    import torch
    lens = [1, 17, 300, 0, 129, 64, 65, 513]
    say("fp8 varlen", causal)
    q8, k8, v8, cu_q, cu_k, ds = W.make_varlen_fp8(lens, lens, 4, 2, 128, seed=33, wid=WID)
    scale = 0.1
    o, lse = fa.attention_fp8(dev_u8(q8), dev_u8(k8), dev_u8(v8), q_descale=ds[0],
                              k_descale=ds[1], v_descale=ds[2], causal=causal, scale=scale,
                              cu_seqlens_q=dev_i32(cu_q), cu_seqlens_k=dev_i32(cu_k),
                              out_dtype=torch.float32)
    torch.cuda.synchronize()
    og, lg = host(o), host(lse)
    for s in range(len(lens)):
        a, e = int(cu_q[s]), int(cu_q[s + 1])
        if e == a:
            continue
        check(og[a:e][None], lg[a:e][None], q8[a:e][None], k8[cu_k[s]:cu_k[s + 1]][None],
              v8[cu_k[s]:cu_k[s + 1]][None], ds, scale, causal, False, f"seq {s}", rms=False)


@pytest.mark.parametrize("causal", [False, True])
def test_fp8_full_size_sampled_heads(fa, causal):
    """The FP8 bench launch: B=4, H=16, N=2048, d=128, checked on whole
    sampled (sequence, head) slices."""
    import torch
    w = W.WORKLOADS[2]
    say("fp8 full size", causal)
    q8, k8, v8, ds = W.make_fixed_fp8(w.batch, w.heads_q, w.heads_kv, w.seqlen_q, w.seqlen_k,
                                      w.head_dim, seed=0, wid=WID + 1)
    o, lse = fa.attention_fp8(dev_u8(q8), dev_u8(k8), dev_u8(v8), q_descale=ds[0],
                              k_descale=ds[1], v_descale=ds[2], causal=causal, scale=w.scale,
                              out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    og, lg = host(o), host(lse)
    assert np.isfinite(og).all() and np.isfinite(lg).all()
    for b, h in ((0, 0), (1, 7), (3, 15)):
        check(og[b:b + 1, :, h:h + 1], lg[b:b + 1, :, h:h + 1], q8[b:b + 1, :, h:h + 1],
              k8[b:b + 1, :, h:h + 1], v8[b:b + 1, :, h:h + 1], ds, w.scale, causal, True,
              f"b{b} h{h}")


@pytest.mark.parametrize("causal", [False, True])
def test_fp8_rising_scores_move_the_reference(fa, causal):
    """Scores that grow along the keys make the rows' references move inside
    the pipelined key loop (probabilities rounded to E4M3 stay below 2^8)."""
    import torch
    say("fp8 rising scores", causal)
    q8, k8, v8, ds = W.make_rising_fp8(1, 4, 2, 1100, 128, seed=5, wid=WID)
    scale = 1 / np.sqrt(128)
    o, lse = fa.attention_fp8(dev_u8(q8), dev_u8(k8), dev_u8(v8), q_descale=ds[0],
                              k_descale=ds[1], v_descale=ds[2], causal=causal, scale=scale,
                              out_dtype=torch.float32)
    torch.cuda.synchronize()
    check(host(o), host(lse), q8, k8, v8, ds, scale, causal, False, f"rising causal={causal}")
