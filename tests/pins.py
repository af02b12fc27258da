"""Independent pins for the fp64 oracle.

Each check ties the oracle to something other than itself: a closed form,
an invariant, a textbook reduction, or the literal matrix-product form of
the definition on tiny inputs.  Every check takes the oracle's forward
function as an argument so the mutation test can run the same checks on
deliberately broken copies of the oracle.

The recurrence being pinned (the standard gated delta rule; the pages,
"Super Apriel: One Checkpoint, Many Speeds", gist.science summary section
2a, only say that KDA is recurrent with a per-channel gate and GDN recurrent
with a scalar gate):
    S_t = S_{t-1} Diag(a_t) (I - b_t k_t k_t^T) + b_t v_t k_t^T,  o_t = S_t q_t
"""
from __future__ import annotations

import numpy as np


def _rand(rng, *shape):
    return rng.standard_normal(shape).astype(np.float32)


def _case(rng, B, T, H, Dk, Dv, channel, h0=True, gscale=0.3):
    q = _rand(rng, B, T, H, Dk)
    k = _rand(rng, B, T, H, Dk)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = _rand(rng, B, T, H, Dv)
    beta = (1 / (1 + np.exp(-_rand(rng, B, T, H)))).astype(np.float32)
    gshape = (B, T, H, Dk) if channel else (B, T, H)
    g = (-np.log1p(np.exp(_rand(rng, *gshape))) * gscale).astype(np.float32)
    S0 = (_rand(rng, B, H, Dv, Dk) * 0.5) if h0 else None
    return q, k, v, g, beta, S0


# --------------------------------------------------------------------------
# P1: beta = 0 and a = 1 leave the state unchanged; the output then reduces
# to one library matrix product o_t = scale * S0 q_t.
def pin_identity(fwd):
    rng = np.random.default_rng(1)
    for channel in (False, True):
        q, k, v, g, beta, S0 = _case(rng, 2, 9, 3, 6, 5, channel)
        g[...] = 0.0
        beta[...] = 0.0
        o, ht = fwd(q, k, v, g, beta, h0=S0, scale=0.75)
        assert np.array_equal(ht, S0.astype(np.float64)), "P1 state moved"
        ref = 0.75 * np.einsum("bhij,bthj->bthi", S0.astype(np.float64),
                               q.astype(np.float64))
        np.testing.assert_allclose(o, ref, rtol=0, atol=1e-12)


# --------------------------------------------------------------------------
# P2: a = 1, beta = 1 and orthonormal keys turn the state into an exact
# associative memory: reading with q_t = k_t returns v_t, and the final state
# maps every stored key to its value (S_T = sum_s v_s k_s^T from S0 = 0).
def pin_orthonormal_retrieval(fwd):
    rng = np.random.default_rng(2)
    Dk, Dv, T = 16, 7, 12
    for channel in (False, True):
        Qm, _ = np.linalg.qr(rng.standard_normal((Dk, Dk)))
        keys = Qm[:T].astype(np.float32)                 # orthonormal rows
        k = keys[None, :, None, :].copy()                # [1,T,1,Dk]
        q = k.copy()
        v = _rand(rng, 1, T, 1, Dv)
        beta = np.ones((1, T, 1), np.float32)
        g = np.zeros((1, T, 1, Dk) if channel else (1, T, 1), np.float32)
        o, ht = fwd(q, k, v, g, beta, h0=None)
        np.testing.assert_allclose(o, v.astype(np.float64), atol=2e-6)
        S = ht[0, 0]
        kk = keys.astype(np.float64)
        np.testing.assert_allclose(S @ kk.T, v[0, :, 0].T.astype(np.float64),
                                   atol=2e-6)
        np.testing.assert_allclose(S, v[0, :, 0].T.astype(np.float64) @ kk,
                                   atol=2e-6)


# --------------------------------------------------------------------------
# P3: a per-channel gate whose Dk entries are all equal is the scalar gate.
def pin_channel_equals_scalar(fwd):
    rng = np.random.default_rng(3)
    q, k, v, g, beta, S0 = _case(rng, 2, 11, 2, 8, 6, channel=False)
    gc = np.repeat(g[..., None], 8, axis=-1)
    o1, h1 = fwd(q, k, v, g, beta, h0=S0)
    o2, h2 = fwd(q, k, v, gc, beta, h0=S0)
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-13)
    np.testing.assert_allclose(h1, h2, rtol=0, atol=1e-13)


# --------------------------------------------------------------------------
# P4: brute force on T <= 8.  The definition multiplied out as dense matrix
# products, with no recursion shared between time steps:
#   M_t = Diag(a_t) (I - b_t k_t k_t^T)
#   S_t = S0 M_1...M_t + sum_{s<=t} b_s v_s k_s^T M_{s+1}...M_t
#   o_t = scale * S_t q_t
def _brute(q, k, v, g, beta, S0, scale):
    T, Dk = q.shape
    Dv = v.shape[1]
    a = np.exp(g.astype(np.float64))
    if a.ndim == 1:
        a = np.repeat(a[:, None], Dk, axis=1)
    M = [np.diag(a[t]) @ (np.eye(Dk) - beta[t] * np.outer(k[t], k[t]))
         for t in range(T)]

    def prod(lo, hi):  # M_lo ... M_{hi-1}
        P = np.eye(Dk)
        for t in range(lo, hi):
            P = P @ M[t]
        return P

    o = np.zeros((T, Dv))
    S = None
    for t in range(T):
        S = S0 @ prod(0, t + 1)
        for s in range(t + 1):
            S = S + beta[s] * np.outer(v[s], k[s]) @ prod(s + 1, t + 1)
        o[t] = scale * S @ q[t]
    return o, S


def pin_bruteforce(fwd):
    rng = np.random.default_rng(4)
    for channel in (False, True):
        for T in (1, 3, 8):
            q, k, v, g, beta, S0 = _case(rng, 1, T, 1, 5, 4, channel,
                                         gscale=0.7)
            k *= 1.3  # keys need not be unit norm for the definition
            o, ht = fwd(q, k, v, g, beta, h0=S0, scale=1.25)
            f = lambda x: x[0, :, 0].astype(np.float64)  # noqa: E731
            ob, Sb = _brute(f(q), f(k), f(v), g[0, :, 0].astype(np.float64),
                            beta[0, :, 0].astype(np.float64),
                            S0[0, 0].astype(np.float64), 1.25)
            np.testing.assert_allclose(o[0, :, 0], ob, rtol=0, atol=1e-12)
            np.testing.assert_allclose(ht[0, 0], Sb, rtol=0, atol=1e-12)


# --------------------------------------------------------------------------
# P5: for fixed q, k, beta, g the map (S0, V) -> (O, S_T) is linear.
def pin_linearity(fwd):
    rng = np.random.default_rng(5)
    for channel in (False, True):
        q, k, v1, g, beta, S1 = _case(rng, 1, 10, 2, 6, 6, channel)
        _, _, v2, _, _, S2 = _case(rng, 1, 10, 2, 6, 6, channel)
        al, be = 0.5, -1.5
        oa, ha = fwd(q, k, v1, g, beta, h0=S1)
        ob, hb = fwd(q, k, v2, g, beta, h0=S2)
        oc, hc = fwd(q, k, al * v1 + be * v2, g, beta, h0=al * S1 + be * S2)
        np.testing.assert_allclose(oc, al * oa + be * ob, atol=1e-6)
        np.testing.assert_allclose(hc, al * ha + be * hb, atol=1e-6)


# --------------------------------------------------------------------------
# P6: resume.  Running T tokens equals running T1, then T - T1 starting from
# the state the first call returned.
def pin_resume(fwd):
    rng = np.random.default_rng(6)
    for channel in (False, True):
        T = 37
        q, k, v, g, beta, S0 = _case(rng, 2, T, 2, 6, 5, channel)
        o, ht = fwd(q, k, v, g, beta, h0=S0)
        for T1 in (1, 16, 23, 36):
            sl1 = (slice(None), slice(0, T1))
            sl2 = (slice(None), slice(T1, T))
            oa, ha = fwd(q[sl1], k[sl1], v[sl1], g[sl1], beta[sl1], h0=S0)
            ob, hb = fwd(q[sl2], k[sl2], v[sl2], g[sl2], beta[sl2],
                         h0=ha.astype(np.float32))
            # the hand-off state is rounded to fp32 once
            np.testing.assert_allclose(np.concatenate([oa, ob], 1), o,
                                       atol=1e-5)
            np.testing.assert_allclose(hb, ht, atol=1e-5)


# --------------------------------------------------------------------------
# P7: packed variable-length batch equals separate calls per sequence; no
# state crosses a cu_seqlens boundary (including empty sequences).
def pin_varlen(fwd):
    rng = np.random.default_rng(7)
    lens = [5, 0, 13, 1, 8]
    cu = np.concatenate([[0], np.cumsum(lens)])
    for channel in (False, True):
        Tt = int(cu[-1])
        q, k, v, g, beta, _ = _case(rng, 1, Tt, 3, 6, 4, channel)
        S0 = _rand(rng, len(lens), 3, 4, 6)
        sq = lambda x: x[0]  # noqa: E731
        o, ht = fwd(sq(q), sq(k), sq(v), sq(g), sq(beta), h0=S0, cu_seqlens=cu)
        for n, L in enumerate(lens):
            sl = (slice(None), slice(int(cu[n]), int(cu[n + 1])))
            on, hn = fwd(q[sl], k[sl], v[sl], g[sl], beta[sl], h0=S0[n:n + 1])
            np.testing.assert_array_equal(o[cu[n]:cu[n + 1]], on[0])
            np.testing.assert_array_equal(ht[n], hn[0])
        # empty sequence: final state is its initial state
        np.testing.assert_array_equal(ht[1], S0[1].astype(np.float64))


# --------------------------------------------------------------------------
# P8: one token from a zero state gives S = b v k^T and o = b v (k.q); with
# a = 0 (g = -inf) the state forgets, so every step is S_t = b_t v_t k_t^T.
def pin_single_token_and_forget(fwd):
    rng = np.random.default_rng(8)
    for channel in (False, True):
        q, k, v, g, beta, _ = _case(rng, 1, 6, 1, 7, 3, channel, h0=False)
        k *= 0.8
        f64 = lambda x: x.astype(np.float64)  # noqa: E731
        o, ht = fwd(q[:, :1], k[:, :1], v[:, :1], g[:, :1], beta[:, :1])
        b0 = f64(beta[0, 0, 0])
        np.testing.assert_allclose(
            ht[0, 0], b0 * np.outer(f64(v[0, 0, 0]), f64(k[0, 0, 0])),
            rtol=0, atol=1e-13)
        np.testing.assert_allclose(
            o[0, 0, 0], b0 * f64(v[0, 0, 0]) * (f64(k[0, 0, 0]) @ f64(q[0, 0, 0])),
            rtol=0, atol=1e-12)
        g[...] = -np.inf
        S0 = _rand(rng, 1, 1, 3, 7)
        o, ht = fwd(q, k, v, g, beta, h0=S0)
        for t in range(6):
            St = f64(beta[0, t, 0]) * np.outer(f64(v[0, t, 0]), f64(k[0, t, 0]))
            np.testing.assert_allclose(o[0, t, 0], St @ f64(q[0, t, 0]),
                                       rtol=0, atol=1e-12)
        np.testing.assert_allclose(ht[0, 0], St, rtol=0, atol=1e-13)


# --------------------------------------------------------------------------
# P9: scalar gate with beta = 0: pure decay, S_t = (prod_{s<=t} alpha_s) S0.
def pin_pure_decay(fwd):
    rng = np.random.default_rng(9)
    q, k, v, g, beta, S0 = _case(rng, 1, 12, 2, 5, 6, channel=False)
    beta[...] = 0.0
    o, ht = fwd(q, k, v, g, beta, h0=S0)
    cum = np.exp(np.cumsum(g[0].astype(np.float64), axis=0))  # [T,H]
    for h in range(2):
        S = S0[0, h].astype(np.float64)
        ref = cum[:, h, None] * (q[0, :, h].astype(np.float64) @ S.T)
        np.testing.assert_allclose(o[0, :, h], ref, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(ht[0, h], cum[-1, h] * S, rtol=1e-12,
                                   atol=1e-14)


# --------------------------------------------------------------------------
# Worked example by hand (Dk = Dv = 2, T = 2, dyadic values so the answer is
# exact).  Channel gate a_2 = (1/2, 1/4), scalar gate a_2 = 1/2.
#   S0 = [[1, 2], [0, 1]]
#   t=1: k=(1,0) v=(2,3) b=1/2 a=1 q=(1,0)
#        S' = S0, S'k = (1, 0), u = b(v - S'k) = (1/2, 3/2)
#        S1 = S0 + u k^T = [[3/2, 2], [3/2, 1]],  o1 = S1 q = (3/2, 3/2)
#   t=2: k=(3/4,1/2) v=(1,-1) b=1 q=(1,1)
#     channel, a=(1/2,1/4): S' = [[3/4, 1/2], [3/4, 1/4]]
#        S'k = (13/16, 11/16), u = (3/16, -27/16)
#        S2 = S' + u k^T = [[57/64, 19/32], [-33/64, -19/32]]
#        o2 = S2 q = (95/64, -71/64)
#     scalar, a=1/2:      S' = [[3/4, 1], [3/4, 1/2]]
#        S'k = (17/16, 13/16), u = (-1/16, -29/16)
#        S2 = [[45/64, 31/32], [-39/64, -13/32]],  o2 = (107/64, -65/64)
def pin_worked_example(fwd):
    S0 = np.array([[[[1, 2], [0, 1]]]], np.float32)
    k = np.array([[[[1, 0]], [[0.75, 0.5]]]], np.float32)
    q = np.array([[[[1, 0]], [[1, 1]]]], np.float32)
    v = np.array([[[[2, 3]], [[1, -1]]]], np.float32)
    beta = np.array([[[0.5], [1.0]]], np.float32)
    cases = {
        True: (np.log(np.array([[[[1, 1]], [[0.5, 0.25]]]], np.float64)),
               [[57 / 64, 19 / 32], [-33 / 64, -19 / 32]], [95 / 64, -71 / 64]),
        False: (np.log(np.array([[[1], [0.5]]], np.float64)),
                [[45 / 64, 31 / 32], [-39 / 64, -13 / 32]], [107 / 64, -65 / 64]),
    }
    for channel, (g, S2, o2) in cases.items():
        o, ht = fwd(q, k, v, g.astype(np.float32), beta, h0=S0)
        # ln(1/2), ln(1/4) are not exact in fp32: allow ~1 ulp of the gate
        np.testing.assert_allclose(o[0, 0, 0], [1.5, 1.5], atol=1e-6)
        np.testing.assert_allclose(o[0, 1, 0], o2, atol=1e-6)
        np.testing.assert_allclose(ht[0, 0], S2, atol=1e-6)


ALL_PINS = [pin_identity, pin_orthonormal_retrieval, pin_channel_equals_scalar,
            pin_bruteforce, pin_linearity, pin_resume, pin_varlen,
            pin_single_token_and_forget, pin_pure_decay, pin_worked_example]
