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
