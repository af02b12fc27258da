"""CPU pins for the oracle's serving forms: several decode tokens per launch
with per-token checkpoints, and states kept in a slot-indexed pool.

Each pin ties the oracle to a closed form of the recurrence
    S_t = S_{t-1} Diag(a_t) (I - b_t k_t k_t^T) + b_t v_t k_t^T,  o_t = S_t q_t
(the standard gated delta rule; "Super Apriel: One Checkpoint, Many Speeds",
gist.science summary section 2a, names the two gate kinds) under an input
choice that makes the answer known, and uses pool slots that differ from
the sequence index, so that a slot map that is ignored, inverted or applied
to the wrong side fails.
"""
import functools

import numpy as np
import pytest

import oracle


def _orthonormal(rng, T, D):
    Qm, _ = np.linalg.qr(rng.standard_normal((D, D)))
    return Qm[:T].astype(np.float32)


# a = 1, beta = 1, orthonormal keys, q_t = k_t, zero initial state: the state
# after token t is sum_{s<=t} v_s k_s^T and every output returns its value.
def pin_tokens_orthonormal(dec):
    rng = np.random.default_rng(21)
    B, n, H, D, P = 3, 5, 2, 8, 6
    slot = np.array([4, 1, 2])
    k = np.stack([np.stack([_orthonormal(rng, n, D) for _ in range(H)], 1)
                  for _ in range(B)])                       # [B,n,H,D]
    q = k.copy()
    v = rng.standard_normal((B, n, H, D)).astype(np.float32)
    beta = np.ones((B, n, H), np.float32)
    for channel in (False, True):
        g = np.zeros((B, n, H, D) if channel else (B, n, H), np.float32)
        pool = rng.standard_normal((P, H, D, D)).astype(np.float32)
        pool[slot] = 0.0
        o, newp, ck = dec(q, k, v, g, beta, pool, slot=slot, checkpoints=True)
        # the keys are orthonormal up to their rounding to float32 (~1e-7)
        np.testing.assert_allclose(o, v, atol=2e-6)
        ref = np.cumsum(np.einsum("bthi,bthj->bthij", v.astype(np.float64),
                                  k.astype(np.float64)), axis=1)
        np.testing.assert_allclose(ck, ref, atol=2e-6)
        assert np.array_equal(newp, pool.astype(np.float64)), "checkpointed call moved the pool"
        o2, newp2, _ = dec(q, k, v, g, beta, pool, slot=slot)
        np.testing.assert_allclose(newp2[slot], ref[:, -1], atol=2e-6)
        rest = np.setdiff1d(np.arange(P), slot)
        assert np.array_equal(newp2[rest], pool[rest].astype(np.float64))


# beta = 0: only the gate acts, S_t = S_0 Diag(prod_{s<=t} a_s) (channel) or
# (prod a_s) S_0 (scalar).  Distinct pool states make every slot traceable;
# an idle sequence (slot -1) leaves its outputs unwritten and the pool as is.
def pin_tokens_pure_decay(dec):
    rng = np.random.default_rng(22)
    B, n, H, D, P = 4, 3, 2, 6, 7
    slot = np.array([5, -1, 0, 3])
    act = np.array([0, 2, 3])
    q = rng.standard_normal((B, n, H, D)).astype(np.float32)
    k = rng.standard_normal((B, n, H, D)).astype(np.float32)
    v = rng.standard_normal((B, n, H, D)).astype(np.float32)
    beta = np.zeros((B, n, H), np.float32)
    pool = rng.standard_normal((P, H, D, D)).astype(np.float32)
    for channel in (False, True):
        g = (-rng.uniform(0, 0.5, (B, n, H, D) if channel else (B, n, H))).astype(np.float32)
        cum = np.exp(np.cumsum(g.astype(np.float64), axis=1))
        S0 = pool[np.where(slot >= 0, slot, 0)].astype(np.float64)   # [B,H,D,D]
        if channel:
            ref = S0[:, None] * cum[:, :, :, None, :]
        else:
            ref = S0[:, None] * cum[:, :, :, None, None]
        o, newp, ck = dec(q, k, v, g, beta, pool, slot=slot, checkpoints=True, scale=0.5)
        np.testing.assert_allclose(ck[act], ref[act], rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(
            o[act], 0.5 * np.einsum("bthij,bthj->bthi", ref[act], q[act].astype(np.float64)),
            rtol=1e-12, atol=1e-12)
        assert np.isnan(o[1]).all() and np.isnan(ck[1]).all()
        _, newp2, _ = dec(q, k, v, g, beta, pool, slot=slot)
        np.testing.assert_allclose(newp2[slot[act]], ref[act, -1], rtol=1e-13, atol=1e-13)
        rest = np.setdiff1d(np.arange(P), slot[act])
        assert np.array_equal(newp2[rest], pool[rest].astype(np.float64))


# Packed prefill through the pool, beta = 0: sequence n's final state is its
# start state (pool[h0_slot[n]], or zeros for -1) times the product of its
# gates, stored at ht_slot[n]; an empty sequence copies its start state; a
# sequence with ht_slot -1 stores nothing; untouched slots keep their bytes.
def pin_pool_prefill_pure_decay(fwd_pool):
    rng = np.random.default_rng(23)
    lens = [5, 0, 9, 4]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    Tt, H, D, P = int(cu[-1]), 2, 6, 6
    h0_slot = np.array([2, 0, -1, 5])
    ht_slot = np.array([2, 4, 1, -1])
    q = rng.standard_normal((Tt, H, D)).astype(np.float32)
    k = rng.standard_normal((Tt, H, D)).astype(np.float32)
    v = rng.standard_normal((Tt, H, D)).astype(np.float32)
    beta = np.zeros((Tt, H), np.float32)
    pool = rng.standard_normal((P, H, D, D)).astype(np.float32)
    for channel in (False, True):
        g = (-rng.uniform(0, 0.4, (Tt, H, D) if channel else (Tt, H))).astype(np.float32)
        o, newp = fwd_pool(q, k, v, g, beta, cu, pool, h0_slot, ht_slot, scale=1.0)
        exp_pool = pool.astype(np.float64).copy()
        for i in range(len(lens)):
            S = (pool[h0_slot[i]].astype(np.float64) if h0_slot[i] >= 0
                 else np.zeros((H, D, D)))
            for t in range(cu[i], cu[i + 1]):
                a = np.exp(g[t].astype(np.float64))
                S = S * (a[:, None, :] if channel else a[:, None, None])
                np.testing.assert_allclose(o[t], np.einsum("hij,hj->hi", S, q[t]),
                                           rtol=1e-12, atol=1e-12)
            if ht_slot[i] >= 0:
                exp_pool[ht_slot[i]] = S
        np.testing.assert_allclose(newp, exp_pool, rtol=1e-13, atol=1e-13)
        assert np.array_equal(newp[[0, 3, 5]], pool[[0, 3, 5]].astype(np.float64))


SERVING_PINS = [pin_tokens_orthonormal, pin_tokens_pure_decay]


@pytest.mark.parametrize("pin", SERVING_PINS, ids=lambda f: f.__name__)
def test_oracle_decode_tokens_pin(pin, oracle_lib):
    pin(functools.partial(oracle.decode_tokens, lib=oracle_lib))


def test_oracle_pool_prefill_pin(oracle_lib):
    pin_pool_prefill_pure_decay(functools.partial(oracle.forward_pool, lib=oracle_lib))


# The pins notice a slot map that is dropped or applied to the wrong side.
def test_serving_pins_catch_slot_mistakes(oracle_lib):
    def ignore_slot(*a, slot=None, **kw):
        return oracle.decode_tokens(*a, slot=None, lib=oracle_lib, **kw)

    def shifted_slot(*a, slot=None, **kw):
        s = np.asarray(slot)
        return oracle.decode_tokens(*a, slot=np.where(s >= 0, (s + 1) % 6, s),
                                    lib=oracle_lib, **kw)

    for pin in SERVING_PINS:
        for bad in (ignore_slot, shifted_slot):
            with pytest.raises(AssertionError):
                pin(bad)

    def swapped(q, k, v, g, beta, cu, pool, h0_slot, ht_slot, **kw):
        return oracle.forward_pool(q, k, v, g, beta, cu, pool, ht_slot, h0_slot,
                                   lib=oracle_lib, **kw)
    with pytest.raises(AssertionError):
        pin_pool_prefill_pure_decay(swapped)


# --------------------------------------------------------------------------
# Fused input preprocessing: q and k normalised per token, beta from its
# logit by the logistic function, g = -c softplus(logit).

def _fused(q, k, v, xg, xb, c, **kw):
    qh, kh, g, beta = oracle.preprocess(q, k, xg, xb, c)
    return oracle.forward(qh, kh, v, g, beta, **kw)


# One token worked by hand (Dk = Dv = 2): q = (3, 4) -> (0.6, 0.8);
# k = (0, 2) -> (0, 1); beta logit 0 -> 1/2; gate logit 0 with c = 1 ->
# g = -ln 2, a = 1/2.  From S0 = [[1, 2], [3, 4]]: S' = S0 / 2,
# S'k = (1, 2), u = (5 - 1, 6 - 2) / 2 = (2, 2), S1 = [[0.5, 3], [1.5, 4]],
# o = S1 q = (2.7, 4.1).
def pin_fused_worked_example(fused):
    q = np.array([[[[3.0, 4.0]]]], np.float32)
    k = np.array([[[[0.0, 2.0]]]], np.float32)
    v = np.array([[[[5.0, 6.0]]]], np.float32)
    S0 = np.array([[[[1.0, 2.0], [3.0, 4.0]]]], np.float32)
    for channel in (False, True):
        xg = np.zeros((1, 1, 1, 2) if channel else (1, 1, 1), np.float32)
        xb = np.zeros((1, 1, 1), np.float32)
        o, ht = fused(q, k, v, xg, xb, 1.0, h0=S0)
        # the 1e-6 inside the norms moves the result by about 1e-7
        np.testing.assert_allclose(o[0, 0, 0], [2.7, 4.1], atol=1e-6)
        np.testing.assert_allclose(ht[0, 0], [[0.5, 3.0], [1.5, 4.0]], atol=1e-6)


# Scale invariance: multiplying q_t or k_t by any positive number changes
# nothing once they are normalised.
def pin_fused_scale_invariance(fused):
    rng = np.random.default_rng(24)
    B, T, H, D = 2, 7, 2, 8
    q = rng.standard_normal((B, T, H, D)).astype(np.float32)
    k = rng.standard_normal((B, T, H, D)).astype(np.float32)
    v = rng.standard_normal((B, T, H, D)).astype(np.float32)
    xb = rng.standard_normal((B, T, H)).astype(np.float32)
    S0 = (0.1 * rng.standard_normal((B, H, D, D))).astype(np.float32)
    sq = rng.uniform(0.5, 4.0, (B, T, H, 1)).astype(np.float32)
    sk = rng.uniform(0.5, 4.0, (B, T, H, 1)).astype(np.float32)
    for channel in (False, True):
        xg = rng.standard_normal((B, T, H, D) if channel else (B, T, H)).astype(np.float32)
        o1, h1 = fused(q, k, v, xg, xb, 0.3, h0=S0)
        o2, h2 = fused(q * sq, k * sk, v, xg, xb, 0.3, h0=S0)
        np.testing.assert_allclose(o2, o1, rtol=1e-5, atol=1e-6)
        np.testing.assert_allclose(h2, h1, rtol=1e-5, atol=1e-6)


# Saturated logits reduce the fused form to the retrieval closed form:
# beta logit 40 -> beta = 1 (to 4e-18), gate logit -40 -> a = 1 (to 4e-18),
# keys that are orthonormal rows times 3, q_t = k_t / 2: o_t = v_t.
def pin_fused_saturated_retrieval(fused):
    rng = np.random.default_rng(25)
    D, T = 16, 10
    Qm, _ = np.linalg.qr(rng.standard_normal((D, D)))
    keys = (3.0 * Qm[:T]).astype(np.float32)[None, :, None, :]
    v = rng.standard_normal((1, T, 1, D)).astype(np.float32)
    xb = np.full((1, T, 1), 40.0, np.float32)
    for channel in (False, True):
        xg = np.full((1, T, 1, D) if channel else (1, T, 1), -40.0, np.float32)
        o, ht = fused(keys * 0.5, keys, v, xg, xb, 1.0)
        np.testing.assert_allclose(o, v.astype(np.float64), atol=2e-6)


# Gate alone: beta logit -40 (beta = 4e-18), gate logit 0 with c = 0.5 gives
# a = 2^-0.5 per token, so S_t = 2^{-t/2} S0 and o_t = S_t q_hat_t.
def pin_fused_pure_decay(fused):
    rng = np.random.default_rng(26)
    B, T, H, D = 2, 6, 3, 8
    q = rng.standard_normal((B, T, H, D)).astype(np.float32)
    k = rng.standard_normal((B, T, H, D)).astype(np.float32)
    v = rng.standard_normal((B, T, H, D)).astype(np.float32)
    xb = np.full((B, T, H), -40.0, np.float32)
    S0 = rng.standard_normal((B, H, D, D)).astype(np.float32)
    qh = q.astype(np.float64) / np.linalg.norm(q.astype(np.float64), axis=-1, keepdims=True)
    for channel in (False, True):
        xg = np.zeros((B, T, H, D) if channel else (B, T, H), np.float32)
        o, ht = fused(q, k, v, xg, xb, 0.5, h0=S0)
        # g is rounded to float32 once per token: a relative 1e-8 over six tokens
        np.testing.assert_allclose(ht, S0 * 2.0 ** (-T / 2), rtol=1e-7, atol=1e-12)
        for t in range(T):
            St = S0.astype(np.float64) * 2.0 ** (-(t + 1) / 2)
            np.testing.assert_allclose(o[:, t], np.einsum("bhij,bhj->bhi", St, qh[:, t]),
                                       rtol=1e-6, atol=1e-6)


FUSED_PINS = [pin_fused_worked_example, pin_fused_scale_invariance,
              pin_fused_saturated_retrieval, pin_fused_pure_decay]


@pytest.mark.parametrize("pin", FUSED_PINS, ids=lambda f: f.__name__)
def test_oracle_fused_pin(pin, oracle_lib):
    pin(functools.partial(_fused, lib=oracle_lib))


# Plausible mistakes in the preprocessing fail a pin: no normalisation,
# the logistic function of the wrong sign, softplus without its minus sign,
# a gate scale that is dropped, and the norm taken over the wrong axis.
@pytest.mark.parametrize("mistake", ["no_norm", "sigmoid_sign", "softplus_sign",
                                     "drop_scale", "norm_axis"])
def test_fused_pins_catch_mistakes(mistake, oracle_lib):
    def bad(q, k, v, xg, xb, c, **kw):
        qh, kh, g, beta = oracle.preprocess(q, k, xg, xb, c)
        if mistake == "no_norm":
            qh, kh = np.asarray(q, np.float32), np.asarray(k, np.float32)
        elif mistake == "sigmoid_sign":
            beta = (1 - beta).astype(np.float32)
        elif mistake == "softplus_sign":
            g = (-g).astype(np.float32)
        elif mistake == "drop_scale":
            g = (g / c).astype(np.float32)
        elif mistake == "norm_axis":
            kf = np.asarray(k, np.float64)
            kh = (kf / np.sqrt((kf * kf).sum(-2, keepdims=True) + 1e-6)).astype(np.float32)
        return oracle.forward(qh, kh, v, g, beta, lib=oracle_lib, **kw)
    failed = 0
    for pin in FUSED_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(bad)
        except AssertionError:
            failed += 1
    assert failed >= 1, "no pin caught %s" % mistake
