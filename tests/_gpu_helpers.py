"""Shared helpers of the GPU tests: move generator outputs to the device and
compare device results with the fp64 oracle."""
import sys

import numpy as np

O_TOL = 1e-2     # max-abs error on O (fp32 output), bf16 inputs, fp32 accumulation
LSE_TOL = 1e-3   # max-abs error on the natural-log LSE


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def dev_bf16(bits):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def dev_i32(x):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).cuda()


def host(t):
    import torch
    return t.float().cpu().numpy().astype(np.float64) if t.dtype != torch.float64 else t.cpu().numpy()


def bf16_half_ulp(x):
    """Half a bfloat16 ulp at |x| (the rounding error bound of a bf16 store)."""
    ax = np.maximum(np.abs(x), np.finfo(np.float32).tiny)
    return np.exp2(np.floor(np.log2(ax)) - 8)


def check_o(o_gpu, o_ref, bf16_out, what=""):
    o_gpu = np.asarray(o_gpu, np.float64)
    assert np.isfinite(o_gpu).all(), f"{what}: non-finite O"
    err = np.abs(o_gpu - o_ref)
    tol = O_TOL + (bf16_half_ulp(o_ref) if bf16_out else 0.0)
    bad = err > tol
    assert not bad.any(), (f"{what}: O max-abs {err.max():.3e} (worst excess "
                           f"{(err - tol).max():.3e}) at {np.argwhere(bad)[:3].tolist()}")
    return float(err.max())


def check_lse(l_gpu, l_ref, what=""):
    l_gpu = np.asarray(l_gpu, np.float64)
    fin = np.isfinite(l_ref)
    assert np.array_equal(np.isfinite(l_gpu), fin), f"{what}: -inf pattern of LSE differs"
    assert np.array_equal(np.isneginf(l_gpu), np.isneginf(l_ref)), f"{what}: LSE -inf rows"
    err = np.abs(l_gpu[fin] - l_ref[fin]).max(initial=0.0)
    assert err <= LSE_TOL, f"{what}: LSE max-abs {err:.3e}"
    return float(err)
