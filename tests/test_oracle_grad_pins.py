"""Pins of the gradient oracle (oracle/grad.py) that do not use its code:
central finite differences of the forward oracle, torch autograd in fp64,
and closed forms that follow from the definition."""
import numpy as np
import pytest
import torch

import oracle
import oracle.grad as OG


def rand(shape, rng, scale=1.0):
    return rng.standard_normal(shape) * scale


def loss(q, k, v, do, scale, causal):
    o, _ = oracle.attention(q, k, v, scale, causal)
    return float((o * do).sum())


def finite_difference_grad(q, k, v, do, scale, causal, h=1e-6):
    """Central differences of <dO, O(Q, K, V)>, one input element at a time."""
    out = []
    for which in range(3):
        args = [q.copy(), k.copy(), v.copy()]
        x = args[which]
        g = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            x0 = x[idx]
            x[idx] = x0 + h
            lp = loss(*args, do, scale, causal)
            x[idx] = x0 - h
            lm = loss(*args, do, scale, causal)
            x[idx] = x0
            g[idx] = (lp - lm) / (2 * h)
        out.append(g)
    return out


FD_CASES = [
    # (B, Nq, Nk, Hq, Hkv, d, causal)
    (1, 3, 5, 2, 1, 4, False),
    (1, 3, 5, 2, 1, 4, True),    # Lq < Lk, bottom-right causal
    (1, 4, 3, 2, 2, 3, True),    # Lq > Lk: the first row sees no key
    (2, 2, 2, 1, 1, 2, True),
]


def _fd_pin():
    rng = np.random.default_rng(11)
    for (bsz, nq, nk, hq, hkv, d, causal) in FD_CASES:
        q, k, v = rand((bsz, nq, hq, d), rng), rand((bsz, nk, hkv, d), rng), rand((bsz, nk, hkv, d), rng)
        do = rand((bsz, nq, hq, d), rng)
        scale = 0.7
        got = oracle.attention_grad(q, k, v, do, scale, causal)
        ref = finite_difference_grad(q, k, v, do, scale, causal)
        for g, r in zip(got, ref):
            np.testing.assert_allclose(g, r, rtol=1e-6, atol=1e-8)


def torch_grads(q, k, v, do, scale, causal):
    """torch autograd of scaled_dot_product_attention in fp64 on the CPU; K/V
    heads repeated for grouped heads, an explicit bottom-right causal mask."""
    g = q.shape[2] // k.shape[2]
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    kk = tk.repeat_interleave(g, dim=2).transpose(1, 2)
    vv = tv.repeat_interleave(g, dim=2).transpose(1, 2)
    nq, nk = q.shape[1], k.shape[1]
    mask = None
    if causal:
        mask = torch.arange(nk)[None, :] <= torch.arange(nq)[:, None] + (nk - nq)
    o = torch.nn.functional.scaled_dot_product_attention(tq.transpose(1, 2), kk, vv,
                                                         attn_mask=mask, scale=scale)
    (o.transpose(1, 2) * torch.tensor(do)).sum().backward()
    return tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy()


def _torch_pin():
    rng = np.random.default_rng(12)
    for (bsz, nq, nk, hq, hkv, d, causal) in [(2, 37, 37, 4, 2, 16, False),
                                             (2, 37, 37, 4, 2, 16, True),
                                             (1, 20, 45, 6, 3, 8, True)]:
        q, k, v = rand((bsz, nq, hq, d), rng), rand((bsz, nk, hkv, d), rng), rand((bsz, nk, hkv, d), rng)
        do = rand((bsz, nq, hq, d), rng)
        scale = 1.0 / np.sqrt(d)
        got = oracle.attention_grad(q, k, v, do, scale, causal)
        ref = torch_grads(q, k, v, do, scale, causal)
        for g, r in zip(got, ref):
            np.testing.assert_allclose(g, r, rtol=1e-9, atol=1e-11)


def _closed_form_pin():
    """Shifting every key by one vector adds q_i·c to a whole score row, which
    the softmax ignores: the key gradients of each head sum to zero over the
    keys.  Rows of P sum to one: the value gradients summed over the keys
    equal dO summed over the rows that see a key.  Constant V makes O
    independent of Q and K: dQ = dK = 0."""
    rng = np.random.default_rng(13)
    bsz, nq, nk, hq, hkv, d = 2, 30, 30, 4, 2, 8
    q, k, v = rand((bsz, nq, hq, d), rng), rand((bsz, nk, hkv, d), rng), rand((bsz, nk, hkv, d), rng)
    do = rand((bsz, nq, hq, d), rng)
    for causal in (False, True):
        dq, dk, dv = oracle.attention_grad(q, k, v, do, 0.4, causal)
        np.testing.assert_allclose(dk.sum(axis=1), 0.0, atol=1e-11)
        g = hq // hkv
        want = do.reshape(bsz, nq, hkv, g, d).sum(axis=(1, 3))
        np.testing.assert_allclose(dv.sum(axis=1), want, atol=1e-11)
        vc = np.full_like(v, -1.25)
        dq0, dk0, _ = oracle.attention_grad(q, k, vc, do, 0.4, causal)
        np.testing.assert_allclose(dq0, 0.0, atol=1e-12)
        np.testing.assert_allclose(dk0, 0.0, atol=1e-12)


def _varlen_pin():
    """Packed sequences give each sequence's fixed-length gradients."""
    rng = np.random.default_rng(14)
    lens = [5, 1, 9, 0, 4]
    cu = np.concatenate([[0], np.cumsum(lens)])
    hq, hkv, d = 4, 2, 8
    q, k, v = rand((cu[-1], hq, d), rng), rand((cu[-1], hkv, d), rng), rand((cu[-1], hkv, d), rng)
    do = rand((cu[-1], hq, d), rng)
    for causal in (False, True):
        dq, dk, dv = oracle.attention_grad_varlen(q, k, v, do, cu, cu, 0.5, causal)
        for s in range(len(lens)):
            a, b = cu[s], cu[s + 1]
            rq, rk, rv = oracle.attention_grad(q[None, a:b], k[None, a:b], v[None, a:b],
                                               do[None, a:b], 0.5, causal)
            np.testing.assert_allclose(dq[a:b], rq[0], atol=1e-13)
            np.testing.assert_allclose(dk[a:b], rk[0], atol=1e-13)
            np.testing.assert_allclose(dv[a:b], rv[0], atol=1e-13)


GRAD_PINS = {"finite_differences": _fd_pin, "torch_autograd": _torch_pin,
             "closed_forms": _closed_form_pin, "varlen": _varlen_pin}


@pytest.mark.parametrize("name", sorted(GRAD_PINS))
def test_gradient_pin(name):
    GRAD_PINS[name]()


# mistakes planted in the gradient oracle; every one must fail a pin
def _no_row_term(p, dp):
    return p * dp


def _sign_flip(p, dp):
    return p * ((p * dp).sum(axis=1, keepdims=True) - dp)


def _dq_no_scale(ds, kh, scale):
    return ds @ kh


def _dk_from_p(ds, qh, scale):
    # dK from dS without the transpose's row/column roles (square inputs only)
    if ds.shape[0] == ds.shape[1]:
        return scale * (ds @ qh)
    return scale * (ds.T @ qh)


def _dv_unnormalised(p, doh):
    return (p * 2.0).T @ doh


MUTANTS = [("softmax_backward", _no_row_term), ("softmax_backward", _sign_flip),
           ("query_grad", _dq_no_scale), ("key_grad", _dk_from_p),
           ("value_grad", _dv_unnormalised)]


@pytest.mark.parametrize("target,mutant", MUTANTS, ids=[m.__name__ for _, m in MUTANTS])
def test_gradient_mutant_is_caught(monkeypatch, target, mutant):
    monkeypatch.setattr(OG, target, mutant)
    caught = []
    for name, pin in GRAD_PINS.items():
        try:
            pin()
        except AssertionError:
            caught.append(name)
    assert caught, f"mutant {mutant.__name__} passed every gradient pin"
