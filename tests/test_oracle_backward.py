"""CPU pins for the oracle's backward (the vector-Jacobian product of the
recurrence, by fp64 autograd through a token-by-token PyTorch forward):

* that forward equals the C oracle (a separate implementation) to 1e-12;
* central finite differences of that forward equal autograd on a tiny case
  for every input, the gate and the initial state (both gate kinds);
* beta = 0 and a = 1 leave the state at S0, where every gradient has a
  closed form: dq_t = scale S0^T do_t, dh0 = dht + scale sum_t do_t q_t^T,
  dk = dv = 0, dbeta_t = (dS_t k_t).(v_t - S0 k_t) and
  dg_t = sum_i dS_t[i, :] (.) S0[i, :] (summed over channels for a scalar
  gate), with dS_t = dht + scale sum_{s >= t} do_s q_s^T.
(The recurrence: S_t = S_{t-1} Diag(a_t)(I - b_t k_t k_t^T) + b_t v_t k_t^T,
o_t = scale S_t q_t -- the standard gated delta rule behind the pages'
"Super Apriel: One Checkpoint, Many Speeds", gist.science summary 2a.)
"""
import numpy as np
import pytest
import torch

import oracle


def _case(rng, B, T, H, D, channel):
    q = rng.standard_normal((B, T, H, D))
    k = rng.standard_normal((B, T, H, D))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, D))
    g = -rng.uniform(0.05, 0.5, (B, T, H, D) if channel else (B, T, H))
    beta = rng.uniform(0.1, 0.9, (B, T, H))
    h0 = 0.5 * rng.standard_normal((B, H, D, D))
    do = rng.standard_normal((B, T, H, D))
    dht = rng.standard_normal((B, H, D, D))
    return [x.astype(np.float32) for x in (q, k, v, g, beta, h0, do, dht)]


@pytest.mark.parametrize("channel", [False, True])
def test_torch_forward_equals_c_oracle(channel, oracle_lib):
    q, k, v, g, beta, h0, _, _ = _case(np.random.default_rng(31), 2, 9, 2, 6, channel)
    t = lambda x: torch.tensor(x.astype(np.float64))  # noqa: E731
    o, ST = oracle.forward_torch(t(q), t(k), t(v), t(g), t(beta), t(h0), scale=0.8)
    o_ref, ht_ref = oracle.forward(q, k, v, g, beta, h0=h0, scale=0.8, lib=oracle_lib)
    np.testing.assert_allclose(o.numpy(), o_ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(ST.numpy(), ht_ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("channel", [False, True])
def test_backward_matches_finite_differences(channel):
    q, k, v, g, beta, h0, do, dht = _case(np.random.default_rng(32), 1, 5, 1, 3, channel)
    grads = oracle.backward(q, k, v, g, beta, do, h0=h0, dht=dht, scale=0.7)
    xs = [x.astype(np.float64) for x in (q, k, v, g, beta, h0)]

    def loss(vals):
        t = [torch.tensor(x) for x in vals]
        o, ST = oracle.forward_torch(*t[:5], t[5], scale=0.7)
        return float((o.numpy() * do).sum() + (ST.numpy() * dht).sum())

    eps = 1e-6
    for n, x in enumerate(xs):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            plus = [y.copy() for y in xs]
            minus = [y.copy() for y in xs]
            plus[n][idx] += eps
            minus[n][idx] -= eps
            num[idx] = (loss(plus) - loss(minus)) / (2 * eps)
        np.testing.assert_allclose(grads[n], num, rtol=1e-6, atol=1e-7,
                                   err_msg="input %d" % n)


@pytest.mark.parametrize("channel", [False, True])
def test_backward_closed_form_without_writes(channel):
    rng = np.random.default_rng(33)
    q, k, v, g, beta, h0, do, dht = _case(rng, 2, 6, 2, 5, channel)
    g[...] = 0.0
    beta[...] = 0.0
    s = 0.6
    dq, dk, dv, dg, db, dh0 = oracle.backward(q, k, v, g, beta, do, h0=h0, dht=dht, scale=s)
    f = lambda x: x.astype(np.float64)  # noqa: E731
    q, k, v, h0, do, dht = map(f, (q, k, v, h0, do, dht))
    T = q.shape[1]
    np.testing.assert_allclose(dq, s * np.einsum("bhij,bthi->bthj", h0, do), atol=1e-12)
    np.testing.assert_allclose(dh0, dht + s * np.einsum("bthi,bthj->bhij", do, q), atol=1e-12)
    assert np.abs(dk).max() < 1e-12 and np.abs(dv).max() < 1e-12
    for t in range(T):
        dSt = dht + s * np.einsum("bthi,bthj->bhij", do[:, t:], q[:, t:])
        w = v[:, t] - np.einsum("bhij,bhj->bhi", h0, k[:, t])
        np.testing.assert_allclose(db[:, t], np.einsum("bhij,bhj,bhi->bh", dSt, k[:, t], w),
                                   atol=1e-11)
        dgt = np.einsum("bhij,bhij->bhj", dSt, h0)
        np.testing.assert_allclose(dg[:, t], dgt if channel else dgt.sum(-1), atol=1e-11)


# The C oracle's hand-written backward (oracle.backward_c), used where the
# autograd form cannot hold a long sequence's graph in memory, pinned to the
# autograd form above (itself pinned to finite differences and closed forms)
# on fixed and packed batches with both gate kinds, zero gates included.
@pytest.mark.parametrize("channel", [False, True])
def test_c_backward_equals_autograd(channel, oracle_lib):
    q, k, v, g, beta, h0, do, dht = _case(np.random.default_rng(41), 2, 150, 2, 8, channel)
    g[0, 70, 1] = -np.inf                      # a zero gate mid-sequence
    g[1, 5:9] = -7.0                           # a strong decay
    ref = oracle.backward(q, k, v, g, beta, do, h0=h0, dht=dht, scale=0.6)
    got = oracle.backward_c(q, k, v, g, beta, do, h0=h0, dht=dht, scale=0.6, lib=oracle_lib)
    for name, x, r in zip(("dq", "dk", "dv", "dg", "dbeta", "dh0"), got, ref):
        assert x.shape == r.shape, name
        np.testing.assert_allclose(x, r, rtol=1e-9, atol=1e-11, err_msg=name)


@pytest.mark.parametrize("channel", [False, True])
def test_c_backward_packed_equals_per_sequence(channel, oracle_lib):
    """A packed batch (an empty sequence, one token, ragged lengths across
    the checkpoint blocks) equals the autograd form run sequence by
    sequence; without h0 or dht both start from zeros."""
    rng = np.random.default_rng(42)
    lens = [70, 0, 1, 129]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    Tt, H, D = int(cu[-1]), 2, 5
    q, k, v, g, beta, h0, do, dht = _case(rng, 1, Tt, H, D, channel)
    q, k, v, g, beta, do = (x[0] for x in (q, k, v, g, beta, do))
    h0 = 0.5 * rng.standard_normal((len(lens), H, D, D)).astype(np.float32)
    got = oracle.backward_c(q, k, v, g, beta, do, h0=h0, cu_seqlens=cu, scale=0.9,
                            lib=oracle_lib)
    for n, L in enumerate(lens):
        a, b = int(cu[n]), int(cu[n + 1])
        if L == 0:
            assert np.all(got[5][n] == 0)
            continue
        ref = oracle.backward(*(x[a:b][None] for x in (q, k, v, g, beta, do)),
                              h0=h0[n:n + 1], scale=0.9)
        for i in range(5):
            np.testing.assert_allclose(got[i][a:b], ref[i][0], rtol=1e-9, atol=1e-11)
        np.testing.assert_allclose(got[5][n], ref[5][0], rtol=1e-9, atol=1e-11)
