"""Parity of the score-variant forward (fa_fwd_ext: sliding window, ALiBi,
softcap) with the fp64 oracle of oracle/variants.py, through the C ABI (needs
a GPU).  Bound as for the plain forward: max-abs 1e-2 on O (fp32 output; bf16
adds half a bf16 ulp of the exact value) and 1e-3 on the natural-log LSE,
with the -inf pattern of rows without admissible keys equal."""
import numpy as np
import pytest

import oracle.variants as V
import workloads as W
from _gpu_helpers import check_lse, check_o, dev_bf16, dev_i32, host, say

pytestmark = pytest.mark.gpu
WID = 220


@pytest.fixture(scope="module")
def fa():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_attention_84_amd as fa
    fa.load()
    return fa


def slopes(h, batch=None):
    s = 2.0 ** (-8.0 * np.arange(1, h + 1) / h)      # the usual geometric ALiBi slopes
    return s if batch is None else np.stack([s * (1 + 0.1 * b) for b in range(batch)])


CASES = [
    # (B, Nq, Nk, Hq, Hkv, d, causal, window, softcap, alibi)
    (2, 300, 300, 4, 2, 128, False, (64, 64), 0.0, None),
    (2, 300, 300, 4, 2, 128, True, (100, -1), 0.0, None),
    (1, 257, 400, 2, 2, 128, False, (-1, 0), 0.0, None),          # = causal, Lq != Lk
    (1, 200, 200, 2, 1, 64, False, (0, 0), 0.0, None),            # one key per row
    (1, 333, 100, 4, 4, 128, True, (20, 3), 0.0, None),           # early rows see nothing
    (2, 250, 250, 4, 2, 128, False, (-1, -1), 30.0, None),        # softcap only
    (2, 250, 250, 4, 2, 128, True, (-1, -1), 5.0, None),
    (2, 250, 250, 8, 2, 128, True, (-1, -1), 0.0, "head"),        # ALiBi slopes [Hq]
    (2, 250, 300, 8, 2, 64, False, (-1, -1), 0.0, "batch"),       # ALiBi slopes [B, Hq]
    (1, 520, 520, 4, 1, 128, True, (128, -1), 20.0, "head"),      # all three
    (3, 130, 130, 2, 2, 64, False, (16, 16), 10.0, "batch"),
    (1, 300, 300, 2, 2, 128, False, (-1, -1), 0.5, None),         # cap saturates tanh
    (1, 300, 300, 4, 2, 128, True, (-1, -1), 0.0, "steep"),       # slopes up to 32 per key
]


def run(fa, case, out):
    import torch
    bsz, nq, nk, hq, hkv, d, causal, window, cap, alibi = case
    q, k, v = W.make_fixed(bsz, hq, hkv, nq, nk, d, seed=21, wid=WID, k_mult=1.5)
    sl = (None if alibi is None else slopes(hq) if alibi == "head" else
          slopes(hq, bsz) if alibi == "batch" else 64 * slopes(hq))
    scale = 1.0 / np.sqrt(d)
    o, lse = fa.attention(dev_bf16(q), dev_bf16(k), dev_bf16(v), causal=causal, scale=scale,
                          window=window, softcap=cap,
                          alibi_slopes=None if sl is None else torch.from_numpy(
                              sl.astype(np.float32)).cuda(),
                          out_dtype=torch.float32 if out == "f32" else torch.bfloat16)
    torch.cuda.synchronize()
    ref = V.attention_ext(q, k, v, scale, causal, window=window, softcap=cap,
                          alibi=None if sl is None else sl.astype(np.float32))
    return host(o), host(lse), ref


@pytest.mark.parametrize("case", CASES, ids=[str(c) for c in CASES])
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_variants_match_oracle(fa, case, out):
    say("variants", case, out)
    og, lg, (orf, lrf) = run(fa, case, out)
    check_o(og, orf, out == "bf16", str(case))
    check_lse(lg, lrf, str(case))


@pytest.mark.parametrize("causal", [False, True])
def test_varlen_variants_match_oracle(fa, causal):
    import torch
    lens_q = [1, 17, 300, 0, 129, 64, 65]
    say("variants varlen", causal)
    q, k, v, cu_q, cu_k = W.make_varlen(lens_q, lens_q, 4, 2, 128, seed=22, wid=WID)
    sl = slopes(4, len(lens_q)).astype(np.float32)
    o, lse = fa.attention(dev_bf16(q), dev_bf16(k), dev_bf16(v), causal=causal, scale=0.1,
                          cu_seqlens_q=dev_i32(cu_q), cu_seqlens_k=dev_i32(cu_k),
                          window=(40, 40), softcap=15.0,
                          alibi_slopes=torch.from_numpy(sl).cuda(), out_dtype=torch.float32)
    torch.cuda.synchronize()
    orf, lrf = V.attention_ext_varlen(q, k, v, cu_q, cu_k, 0.1, causal, window=(40, 40),
                                      softcap=15.0, alibi=sl)
    check_o(host(o), orf, False, "varlen")
    check_lse(host(lse), lrf, "varlen")


def test_window_covering_everything_equals_the_plain_forward(fa):
    """A window wider than the sequence admits every key: the variant kernel
    must then agree with the plain kernel to rounding.  The two kernels are
    different (64 rows per wave against 32) and round the probabilities to
    bf16 for the P V product against different references, each within half
    a bf16 ulp (2^-9 relative) of p; O = sum p v / sum p then differs by at
    most 2 * 2^-9 * max|v| between them.  Both sum the unrounded fp32 p, so
    their LSEs differ only by fp32 summation order."""
    import torch
    say("variants wide window")
    q, k, v = W.make_fixed(2, 4, 2, 300, 300, 128, seed=23, wid=WID)
    args = (dev_bf16(q), dev_bf16(k), dev_bf16(v))
    a = fa.attention(*args, causal=True, out_dtype=torch.float32)
    b = fa.attention(*args, causal=True, window=(10000, 10000), out_dtype=torch.float32)
    torch.cuda.synchronize()
    v_max = float(np.abs(W.bf16_bits_to_f32(v)).max())
    assert (a[0] - b[0]).abs().max().item() <= 2.0 ** -8 * v_max
    assert (a[1] - b[1]).abs().max().item() < 1e-4


LONG = W.WORKLOADS[3]   # B=1, Hq=32, Hkv=8, N=8192, d=128, causal


def test_full_size_sliding_window_sampled(fa):
    """The bench's sliding-window launch (the long GQA workload with a
    4096-key causal window, ALiBi and a softcap), checked on sampled rows."""
    import torch
    say("variants full size")
    inp = W.make_workload(LONG)
    q, k, v = inp["q"], inp["k"], inp["v"]
    sl = slopes(LONG.heads_q).astype(np.float32)
    o, lse = fa.attention(dev_bf16(q), dev_bf16(k), dev_bf16(v), causal=True, scale=LONG.scale,
                          window=(4095, 0), softcap=30.0,
                          alibi_slopes=torch.from_numpy(sl).cuda(), out_dtype=torch.float32)
    torch.cuda.synchronize()
    og, lg = host(o), host(lse)
    assert np.isfinite(og).all() and np.isfinite(lg).all()
    qf = W.bf16_bits_to_f32(q).astype(np.float64)
    kf = W.bf16_bits_to_f32(k).astype(np.float64)
    vf = W.bf16_bits_to_f32(v).astype(np.float64)
    g = LONG.heads_q // LONG.heads_kv
    for h in (0, 13, 31):
        rows = np.array([0, 1, 4095, 4096, 5000, 8191])
        xo, xl = V.head_attention_ext(qf[0, :, h], kf[0, :, h // g], vf[0, :, h // g], LONG.scale,
                                      True, 4095, 0, 30.0, float(sl[h]))
        check_o(og[0, rows, h], xo[rows], False, f"head {h}")
        check_lse(lg[0, rows, h], xl[rows], f"head {h}")


@pytest.mark.parametrize("causal", [False, True])
def test_varlen_window_only_matches_oracle(fa, causal):
    """A window alone runs on the pipelined forward's local-window instance."""
    import torch
    lens = [1, 17, 300, 0, 129, 64, 65, 513]
    say("window varlen", causal)
    q, k, v, cu_q, cu_k = W.make_varlen(lens, lens, 4, 2, 128, seed=24, wid=WID)
    for window in ((40, 40), (0, -1), (200, 7)):
        o, lse = fa.attention(dev_bf16(q), dev_bf16(k), dev_bf16(v), causal=causal, scale=0.1,
                              cu_seqlens_q=dev_i32(cu_q), cu_seqlens_k=dev_i32(cu_k),
                              window=window, out_dtype=torch.float32)
        torch.cuda.synchronize()
        orf, lrf = V.attention_ext_varlen(q, k, v, cu_q, cu_k, 0.1, causal, window=window)
        check_o(host(o), orf, False, f"varlen {window}")
        check_lse(host(lse), lrf, f"varlen {window}")


def test_full_size_window_only_sampled(fa):
    """The bench's window-only launch: the long GQA workload with a 4096-key
    causal window on the pipelined forward, checked on sampled rows."""
    import torch
    say("window full size")
    inp = W.make_workload(LONG)
    q, k, v = inp["q"], inp["k"], inp["v"]
    o, lse = fa.attention(dev_bf16(q), dev_bf16(k), dev_bf16(v), causal=True, scale=LONG.scale,
                          window=(4095, 0), out_dtype=torch.float32)
    torch.cuda.synchronize()
    og, lg = host(o), host(lse)
    assert np.isfinite(og).all() and np.isfinite(lg).all()
    qf = W.bf16_bits_to_f32(q).astype(np.float64)
    kf = W.bf16_bits_to_f32(k).astype(np.float64)
    vf = W.bf16_bits_to_f32(v).astype(np.float64)
    g = LONG.heads_q // LONG.heads_kv
    rows = np.array([0, 63, 64, 4095, 4096, 4100, 6000, 8191])
    for h in (0, 17, 31):
        xo, xl = V.head_attention_ext(qf[0, :, h], kf[0, :, h // g], vf[0, :, h // g], LONG.scale,
                                      True, 4095, 0, 0.0, 0.0)
        check_o(og[0, rows, h], xo[rows], False, f"head {h}")
        check_lse(lg[0, rows, h], xl[rows], f"head {h}")
