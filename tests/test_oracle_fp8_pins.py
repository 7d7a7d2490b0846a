"""Pins of the FP8 oracle (oracle/fp8.py) to things other than itself: the
E4M3 decoder and rounding against torch's float8_e4m3fn conversion and the
format's published landmark values, attention of FP8 inputs against closed
forms, and the probability-rounding bound against rounding instances that a
kernel could produce and a case built to need its subnormal term."""
import numpy as np
import pytest
import torch

import oracle.exact as E
import oracle.fp8 as F
import workloads as W


def torch_decode(codes):
    t = torch.from_numpy(np.asarray(codes, np.uint8).copy())
    return t.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_decoder_matches_torch_on_every_code():
    codes = np.arange(256, dtype=np.uint8)
    ours, ref = F.e4m3_to_f64(codes), torch_decode(codes)
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    assert np.isnan(ours).sum() == 2                       # S.1111.111 only
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])
    assert np.array_equal(np.signbit(ours[ok]), np.signbit(ref[ok]))


@pytest.mark.parametrize("code,value", [(0x38, 1.0), (0x7E, 448.0), (0x01, 2.0 ** -9),
                                        (0x08, 2.0 ** -6), (0x07, 7 * 2.0 ** -9),
                                        (0xB8, -1.0), (0x40, 2.0), (0x3C, 1.5),
                                        (0x00, 0.0)])
def test_decoder_landmarks(code, value):
    # OCP E4M3: bias 7, 3 mantissa bits, largest finite 448, subnormal step 2^-9
    assert F.e4m3_to_f64(np.array([code], np.uint8))[0] == value


def test_negative_zero():
    z = F.e4m3_to_f64(np.array([0x80], np.uint8))[0]
    assert z == 0.0 and np.signbit(z)


def test_rounding_matches_torch():
    rng = np.random.default_rng(5)
    x = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.uniform(-4, 2, 20000),
                        rng.uniform(-448, 448, 2000)])
    # exact midpoints between neighbouring values exercise ties to even
    grid = F.e4m3_to_f64(np.arange(0, 0x7F, dtype=np.uint8))
    x = np.concatenate([x, (grid[1:] + grid[:-1]) / 2, -(grid[1:] + grid[:-1]) / 2])
    x = x[np.abs(x) <= 448.0]
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(F.round_to_e4m3(x), ref)


def test_rounding_is_identity_on_the_grid():
    grid = F.e4m3_to_f64(np.arange(0, 0x7F, dtype=np.uint8))
    assert np.array_equal(F.round_to_e4m3(grid), grid)
    assert np.array_equal(F.round_to_e4m3(-grid), -grid)


def test_rounding_rejects_out_of_range():
    with pytest.raises(ValueError):
        F.round_to_e4m3(np.array([449.0]))


def codes_of(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.float8_e4m3fn).view(
        torch.uint8).numpy()


def test_single_key_returns_its_value_scaled_by_the_v_descale():
    q = codes_of(np.full((1, 3, 2, 8), 2.0))
    k = codes_of(np.full((1, 1, 1, 8), -1.5))
    v = codes_of(np.arange(8, dtype=np.float32).reshape(1, 1, 1, 8))
    o, lse = F.attention_fp8(q, k, v, 0.5, 0.25, 3.0, scale=0.1)
    assert np.allclose(o, 3.0 * np.arange(8.0))
    # LSE of one key is its score: scale * (0.5 * 2) * (0.25 * -1.5) * 8
    assert np.allclose(lse, 0.1 * 1.0 * -0.375 * 8)


def test_equal_scores_average_the_values():
    q = codes_of(np.ones((1, 1, 1, 4)))
    k = codes_of(np.ones((1, 5, 1, 4)))
    v = codes_of(np.arange(20, dtype=np.float32).reshape(1, 5, 1, 4))
    o, lse = F.attention_fp8(q, k, v, 1.0, 1.0, 0.5, scale=1.0)
    # (17 and 19 are not E4M3 values: compare with torch's decoding of the codes)
    assert np.allclose(o[0, 0, 0], 0.5 * torch_decode(v)[0, :, 0].mean(axis=0))
    assert np.allclose(lse, 4.0 + np.log(5.0))


def test_descales_act_like_a_score_scale():
    q, k, v, _ = W.make_fixed_fp8(1, 2, 1, 9, 11, 16, seed=3, wid=900)
    a = F.attention_fp8(q, k, v, 0.5, 0.25, 1.0, scale=0.3, causal=True)
    b = F.attention_fp8(q, k, v, 1.0, 1.0, 1.0, scale=0.3 * 0.125, causal=True)
    assert np.allclose(a[0], b[0]) and np.allclose(a[1], b[1])


def test_fp8_oracle_agrees_with_the_online_recurrence():
    """The plain definition and the oracle's independent tiled online-softmax
    algorithm agree on dequantised FP8 inputs."""
    q, k, v, ds = W.make_fixed_fp8(1, 1, 1, 40, 70, 32, seed=4, wid=900)
    o, lse = F.attention_fp8(q, k, v, *ds, scale=0.2, causal=True)
    qd, kd, vd = (F.dequantize(x, d)[0, :, 0] for x, d in zip((q, k, v), ds))
    o2, lse2 = E.tiled_online_attention(qd, kd, vd, 0.2, 16, 16, causal=True)
    assert np.allclose(o[0, :, 0], o2) and np.allclose(lse[0, :, 0], lse2)


def rounded_instance(q8, k8, v8, ds, scale, causal, shift):
    """O with every probability scaled by 2^shift_i (a kernel's reference
    below the row maximum), rounded to E4M3, scaled back; row sum unrounded."""
    q, k, v = (F.dequantize(x, d) for x, d in zip((q8, k8, v8), ds))
    out = np.zeros(q.shape)
    for h in range(q.shape[2]):
        s = scale * q[0, :, h] @ k[0, :, 0].T
        s = np.where(E.admissible_mask(np.arange(s.shape[0]), s.shape[0], s.shape[1], causal),
                     s, -np.inf)
        w = np.exp(s - s.max(axis=1, keepdims=True))
        pw = F.round_to_e4m3(w * 2.0 ** shift[:, None]) / 2.0 ** shift[:, None]
        out[0, :, h] = pw @ v[0, :, 0] / w.sum(axis=1)[:, None]
    return out


@pytest.mark.parametrize("causal", [False, True])
def test_bound_holds_for_kernel_like_rounding(causal):
    q, k, v, ds = W.make_fixed_fp8(1, 2, 1, 64, 96, 64, seed=6, wid=900)
    scale = 1 / 8
    exact, _ = F.attention_fp8(q, k, v, *ds, scale=scale, causal=causal)
    bound = F.p_rounding_bound(q, k, v, *ds, scale=scale, causal=causal)
    rng = np.random.default_rng(0)
    for _ in range(4):
        shift = rng.uniform(0, 8, size=64)
        err = np.abs(rounded_instance(q, k, v, ds, scale, causal, shift) - exact)
        assert (err <= bound * (1 + 1e-9) + 1e-12).all()
    ref = F.attention_fp8_rounded_p(q, k, v, *ds, scale=scale, causal=causal)
    err = np.abs(ref - exact)
    assert (err <= bound * (1 + 1e-9) + 1e-12).all()
    assert err.max() > 0        # the step does change O
    assert np.sqrt(np.mean(err ** 2)) < 0.25 * bound.max()


def test_bound_needs_its_subnormal_term():
    """One dominant key and many keys with weight about 2^-11: those round to
    zero, and only the subnormal term of the bound covers the lost mass."""
    d = 16
    q = codes_of(np.full((1, 1, 1, d), 1.0))
    kd = np.zeros((1, 401, 1, d), np.float32)
    kd[0, 0, 0, :] = 1.0                              # score 16 * scale
    kd[0, 1:, 0, :] = 1.0 - 11 * np.log(2) / 16       # about 11 ln 2 lower
    k = codes_of(kd)
    v = codes_of(np.ones((1, 401, 1, d)))
    scale = 1.0
    exact, _ = F.attention_fp8(q, k, v, 1.0, 1.0, 1.0, scale=scale)
    ref = F.attention_fp8_rounded_p(q, k, v, 1.0, 1.0, 1.0, scale=scale)
    bound = F.p_rounding_bound(q, k, v, 1.0, 1.0, 1.0, scale=scale)
    err = np.abs(ref - exact)
    assert err.max() > 0.05                            # the rounding loses real mass
    assert (err <= bound).all()
    # without the subnormal term the bound would be too small
    qd, kd2, vd = (F.dequantize(x, 1.0)[0, :, 0] for x in (q, k, v))
    s = qd @ kd2.T
    w = np.exp(s - s.max())
    relative_only = (2.0 ** -4 * w) @ np.abs(vd) / w.sum()
    assert (err > relative_only).any()
