"""Parity of the FP8 forward (fa_fwd_fp8) with the fp64 oracle of
oracle/fp8.py, through the C ABI (needs a GPU).

The result is exact attention of the descaled E4M3 inputs.  The kernel's
error has these sources, each bounded here:
  * the probabilities rounded to E4M3 before the P V product:
    oracle.fp8.p_rounding_bound, elementwise on O;
  * the FP8 matrix core's accumulation.  Probed on gfx950
    (v_mfma_scale_f32_32x32x64_f8f6f4, E4M3 operands, unit scales), it sums
    each run of 8 consecutive contraction terms at one alignment: every
    product is cut toward zero to a multiple of 2^(E - 13), E the exponent
    of the run's largest product (which itself stays exact), and the 8 run
    sums and the accumulator input are added in fp32.  So a 64-term sum is
    off by less than 7 * 2^-13 times the sum over its runs of each run's
    largest product magnitude, plus fp32 rounding.  For a score (two 64-term
    products over head-dim runs of 8) this is
      |ds_ij| <= scale dq dk 7 2^-13 sum_g max_{k in g} |q8_ik| max_{k in g} |k8_jk|,
    which moves the LSE by at most max_j |ds_ij| and O by at most
    (exp(2 max_j |ds_ij|) - 1) max |v|.  For the P V product the same rule
    gives at most 7 2^-13 (1 + 2^-4) max |v| on the normalised O (the run
    maxima of P sum to at most its row sum; P's E4M3 rounding adds 2^-4);
    2^-10 max |v| is used;
  * fp32 arithmetic elsewhere: 2e-3 on O, 1e-3 on the LSE (the bf16 path's
    LSE bound), plus half a bf16 ulp for a bf16 O.
The worst-case bound on the rounding of P is loose, so the RMS of the O error
over a case with many elements is also held to 1.5 times the RMS error of the
oracle's reference rounding (attention_fp8_rounded_p): a misplaced or dropped
key, well inside the worst-case bound, fails that.  One case is built so that
the accumulation term decides: its scores are sums of large products that
cancel beside many small ones that the alignment drops."""
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


RUN = 8          # contraction terms the FP8 matrix core sums at one alignment
RUN_BITS = 13    # bits kept below the leading bit of a run's largest product


def score_err(q8, k8, ds, scale, hq_per_kv=None):
    """Per query row bound on the score error of the FP8 matrix core, shape
    q8.shape[:-1]: max over the keys of scale dq dk 7 2^-RUN_BITS
    sum_g max|q8| max|k8| over each head-dim run g (max over the whole K
    slice of the row's kv head, which covers every admissible key)."""
    q = np.abs(F.e4m3_to_f64(q8))
    k = np.abs(F.e4m3_to_f64(k8))
    b, nq, hq, d = q.shape
    hkv = k.shape[2]
    g = hq // hkv
    qr = q.reshape(b, nq, hq, d // RUN, RUN).max(axis=-1)      # [B, Nq, Hq, runs]
    kr = k.reshape(b, k.shape[1], hkv, d // RUN, RUN).max(axis=-1)
    out = np.zeros((b, nq, hq))
    for bi in range(b):
        for h in range(hq):
            out[bi, :, h] = (qr[bi, :, h] @ kr[bi, :, h // g].T).max(axis=1)
    return (RUN - 1) * 2.0 ** -RUN_BITS * scale * ds[0] * ds[1] * out


def pv_err(v8, ds):
    """Bound on the P V product's accumulation error on the normalised O."""
    return 2.0 ** -10 * np.abs(F.dequantize(v8, ds[2])).max()


def check(o_gpu, lse_gpu, q8, k8, v8, ds, scale, causal, bf16_out, what, rms=True):
    """Compare one fixed-length batch (B, N, H, d) with the oracle."""
    o_ex, l_ex = F.attention_fp8(q8, k8, v8, *ds, scale=scale, causal=causal)
    bound = F.p_rounding_bound(q8, k8, v8, *ds, scale=scale, causal=causal)
    dsc = score_err(q8, k8, ds, scale)
    vmax = np.abs(F.dequantize(v8, ds[2])).max()
    tol = bound + (np.expm1(2 * dsc) * vmax)[..., None] + pv_err(v8, ds) + O_SLACK
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
    (1, 2048, 2048, 2, 1, True),     # 8 causal pairs of full 128-row tiles
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


def cancelling_case(nq=96, nk=320, seed=6):
    """E4M3 inputs whose scores are sums of large products that cancel beside
    small ones the matrix core's alignment drops.  In every head-dim run of 8
    the first term is 16 x (+-16), the sign alternating between runs so that
    these cancel over the row; the other seven terms are 0.125 x 0.21875 =
    0.02734, below the run's alignment step 2^(8 - 13) = 2^-5, on even keys
    only (odd keys have zeros there).  The exact score of an even key is
    scale 112 0.02734 = scale 3.0625, of an odd key 0, so the exact LSE
    exceeds the one of all-zero scores by ln((1 + e^(3.0625 scale)) / 2).
    V is make_fixed_fp8's; the Q and K descales are 1."""
    import torch
    d = 128
    enc = lambda x: torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(  # noqa: E731
        torch.float8_e4m3fn).view(torch.uint8).numpy()
    first = np.arange(d) % RUN == 0
    sign = np.where((np.arange(d) // RUN) % 2 == 0, 1.0, -1.0)
    q = np.where(first, 16.0, 0.125) * np.ones((1, nq, 1, d))
    k = np.where(first, 16.0 * sign, 0.0) * np.ones((1, nk, 1, d))
    k[:, 0::2, :, :] = np.where(first, 16.0 * sign, 0.21875)
    _, _, v8, ds = W.make_fixed_fp8(1, 1, 1, nq, nk, d, seed=seed, wid=WID)
    return enc(q), enc(k), v8, (1.0, 1.0, ds[2])


def test_fp8_cancelling_products_need_the_accumulation_term(fa):
    """The case passes the bound that includes the matrix core's alignment,
    and its LSE error is beyond what exact fp32 accumulation would allow
    (the term decides the outcome)."""
    import torch
    say("fp8 cancelling products")
    q8, k8, v8, ds = cancelling_case()
    scale = 1 / np.sqrt(128)
    o, lse = fa.attention_fp8(dev_u8(q8), dev_u8(k8), dev_u8(v8), q_descale=ds[0],
                              k_descale=ds[1], v_descale=ds[2], causal=False, scale=scale,
                              out_dtype=torch.float32)
    torch.cuda.synchronize()
    og, lg = host(o), host(lse)
    check(og, lg, q8, k8, v8, ds, scale, False, False, "cancelling products", rms=False)
    _, l_ex = F.attention_fp8(q8, k8, v8, *ds, scale=scale, causal=False)
    lerr = np.abs(lg - l_ex).max()
    # exact fp32 accumulation: scores off by rounding only, far below 1e-3
    assert lerr > 10 * LSE_TOL, (
        f"LSE error {lerr:.3e}: the case no longer exercises the accumulation term")
