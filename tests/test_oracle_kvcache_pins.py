"""Pins of the KV-cache step oracle (oracle/kvcache.py), each independent of
the oracle's own code: the rotation against complex multiplication and its
invariants, bfloat16 rounding against the float32 rounding of the input
generator and hand-worked ties, paged storage against contiguous storage, and
the whole step against the plain decode oracle on caches built by direct
assignment in the test."""
import numpy as np
import pytest

import oracle
import oracle.kvcache as KV
import workloads as W


def tables(max_pos, r, base=10000.0):
    """The usual rotary tables: angle t * base^(-2i/r) for pair i."""
    inv = base ** (-np.arange(0, r, 2, dtype=np.float64) / r)
    ang = np.outer(np.arange(max_pos, dtype=np.float64), inv)
    return np.cos(ang), np.sin(ang)


def as_complex_half(x, r):
    return x[..., : r // 2] + 1j * x[..., r // 2: r]


def test_rotation_is_complex_multiplication():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((3, 16))
    ang = rng.uniform(-4, 4, (3, 8))
    y = KV.rotary(x, np.cos(ang), np.sin(ang), 16)
    z = as_complex_half(x, 16) * np.exp(1j * ang)
    np.testing.assert_allclose(y[:, :8], z.real, rtol=0, atol=1e-14)
    np.testing.assert_allclose(y[:, 8:], z.imag, rtol=0, atol=1e-14)


def test_interleaved_is_a_permutation_of_rotate_half():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((5, 12))
    ang = rng.uniform(-3, 3, (5, 6))
    perm = np.r_[np.arange(0, 12, 2), np.arange(1, 12, 2)]   # pairs (2i, 2i+1) -> (i, i+6)
    y_int = KV.rotary(x, np.cos(ang), np.sin(ang), 12, interleaved=True)
    y_half = KV.rotary(x[:, perm], np.cos(ang), np.sin(ang), 12)
    np.testing.assert_allclose(y_int[:, perm], y_half, rtol=0, atol=1e-14)


def test_identity_norms_and_partial_rotation():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((4, 10))
    assert np.array_equal(KV.rotary(x, np.ones((4, 3)), np.zeros((4, 3)), 6), x)
    ang = rng.uniform(-3, 3, (4, 3))
    y = KV.rotary(x, np.cos(ang), np.sin(ang), 6)
    assert np.array_equal(y[:, 6:], x[:, 6:])                       # tail untouched
    np.testing.assert_allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-14)
    pair = y[:, :3] ** 2 + y[:, 3:6] ** 2
    np.testing.assert_allclose(pair, x[:, :3] ** 2 + x[:, 3:6] ** 2, rtol=1e-13)


@pytest.mark.parametrize("interleaved", [False, True])
def test_scores_depend_only_on_relative_position(interleaved):
    rng = np.random.default_rng(3)
    c, s = tables(64, 16)
    q, k = rng.standard_normal(16), rng.standard_normal(16)
    def score(m, n):
        return KV.rotary(q, c[m], s[m], 16, interleaved) @ KV.rotary(k, c[n], s[n], 16, interleaved)
    for m, n, sh in [(5, 3, 7), (0, 9, 20), (30, 30, 11)]:
        assert score(m, n) == pytest.approx(score(m + sh, n + sh), abs=1e-12)
    assert score(4, 4) == pytest.approx(q @ k, abs=1e-12)   # equal positions: plain dot product


def test_bf16_rounding():
    rng = np.random.default_rng(4)
    x32 = (rng.standard_normal(10000) * 10).astype(np.float32)
    ref = W.bf16_bits_to_f32(W.round_f32_to_bf16_bits(x32)).astype(np.float64)
    assert np.array_equal(KV.to_bf16_rne(x32.astype(np.float64)), ref)
    # hand-worked ties: 1 + 2^-8 lies halfway between 1 and 1 + 2^-7 -> even (1);
    # 1 + 3*2^-8 lies halfway between 1 + 2^-7 and 1 + 2^-6 -> even (1 + 2^-6)
    assert KV.to_bf16_rne(1 + 2.0 ** -8) == 1.0
    assert KV.to_bf16_rne(1 + 3 * 2.0 ** -8) == 1 + 2.0 ** -6
    assert KV.to_bf16_rne(-(1 + 2.0 ** -8 + 2.0 ** -30)) == -(1 + 2.0 ** -7)
    assert KV.to_bf16_rne(255.9) == 256.0
    assert np.array_equal(KV.bf16_bits(np.array([1.0, -2.0, 0.5])), np.array([0x3F80, 0xC000, 0x3F00]))


def rand_cache(shape, seed):
    return W.normal_bf16(seed, 901, 0, shape)


def test_step_without_append_or_rotary_is_decode():
    b, hq, hkv, n, d = 3, 8, 2, 50, 64
    q = rand_cache((b, hq, d), 1)
    kc, vc = rand_cache((b, n, hkv, d), 2), rand_cache((b, n, hkv, d), 3)
    lens = np.array([0, 17, 50])
    o, l, k2, v2 = KV.kvcache_step(q, kc, vc, lens, 0.125)
    o_ref, l_ref = oracle.decode(q, kc, vc, lens, 0.125)
    assert np.array_equal(o, o_ref) and np.array_equal(l, l_ref)
    assert np.array_equal(k2, kc) and np.array_equal(v2, vc)


def test_paged_storage_equals_contiguous():
    b, hq, hkv, d, page = 3, 4, 2, 32, 4
    npages = 5                                    # 20 rows per sequence
    q = rand_cache((b, hq, d), 4)
    kc, vc = rand_cache((b, npages * page, hkv, d), 5), rand_cache((b, npages * page, hkv, d), 6)
    lens = np.array([20, 7, 13])
    rng = np.random.default_rng(7)
    phys = rng.permutation(b * npages)           # where each (b, logical page) is stored
    table = phys.reshape(b, npages)
    kp = np.zeros((b * npages, page, hkv, d), np.uint16)
    vp = np.zeros_like(kp)
    for s in range(b):
        for j in range(npages):
            kp[table[s, j]] = kc[s, j * page:(j + 1) * page]
            vp[table[s, j]] = vc[s, j * page:(j + 1) * page]
    o1, l1, _, _ = KV.kvcache_step(q, kc, vc, lens, 0.2)
    o2, l2, _, _ = KV.kvcache_step(q, kp, vp, lens, 0.2, block_table=table, page_size=page)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


@pytest.mark.parametrize("paged", [False, True])
@pytest.mark.parametrize("rot", [None, "half", "interleaved"])
def test_append_with_rotary_matches_decode_on_a_hand_built_cache(paged, rot):
    b, hq, hkv, d, n, page = 2, 4, 2, 32, 12, 4
    q = rand_cache((b, hq, d), 8)
    kn, vn = rand_cache((b, hkv, d), 9), rand_cache((b, hkv, d), 10)
    kc, vc = rand_cache((b, n, hkv, d), 11), rand_cache((b, n, hkv, d), 12)
    lens = np.array([5, 11])
    r = 24 if rot else 0
    c, s = tables(16, 24)
    # the expected cache and query, built here with complex numbers
    kexp, vexp = kc.copy(), vc.copy()
    qexp = W.bf16_bits_to_f32(q).astype(np.float64)
    for i in range(b):
        t = lens[i]
        kf = W.bf16_bits_to_f32(kn[i]).astype(np.float64)
        if rot:
            def rotc(x):
                y = x.copy()
                if rot == "half":
                    z = (x[..., :12] + 1j * x[..., 12:24]) * np.exp(1j * np.arctan2(s[t], c[t]))
                    y[..., :12], y[..., 12:24] = z.real, z.imag
                else:
                    z = (x[..., 0:24:2] + 1j * x[..., 1:24:2]) * np.exp(1j * np.arctan2(s[t], c[t]))
                    y[..., 0:24:2], y[..., 1:24:2] = z.real, z.imag
                return y
            kf = KV.to_bf16_rne(rotc(kf))
            qexp[i] = KV.to_bf16_rne(rotc(qexp[i]))
        kexp[i, t] = KV.bf16_bits(kf)
        vexp[i, t] = vn[i]
    o_ref, l_ref = oracle.decode(KV.bf16_bits(qexp), kexp, vexp, lens + 1, 0.15)
    kw = dict(k_new=kn, v_new=vn)
    if rot:
        kw.update(rotary_cos=c, rotary_sin=s, rotary_dim=r, interleaved=(rot == "interleaved"))
    if paged:
        table = np.array([[2, 0, 5], [4, 1, 3]])
        kp = np.zeros((6, page, hkv, d), np.uint16)
        vp = np.zeros_like(kp)
        for i in range(b):
            for j in range(3):
                kp[table[i, j]] = kc[i, j * page:(j + 1) * page]
                vp[table[i, j]] = vc[i, j * page:(j + 1) * page]
        o, l, k2, v2 = KV.kvcache_step(q, kp, vp, lens, 0.15, block_table=table, page_size=page, **kw)
        for i in range(b):                       # back to logical order
            for j in range(3):
                assert np.array_equal(k2[table[i, j]], kexp[i, j * page:(j + 1) * page])
                assert np.array_equal(v2[table[i, j]], vexp[i, j * page:(j + 1) * page])
    else:
        o, l, k2, v2 = KV.kvcache_step(q, kc, vc, lens, 0.15, **kw)
        assert np.array_equal(k2, kexp) and np.array_equal(v2, vexp)
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l, l_ref, rtol=0, atol=1e-12)
