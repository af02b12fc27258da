"""GPU parity of the serving forms through the C ABI against the fp64
oracle: several decode tokens per launch (with and without per-token
checkpoints), the commit of an accepted prefix, and packed prefill with the
states in a slot-indexed pool.  Small cases compare every element; the
drafted-decode workload (B=256, 4 tokens, H=32, d=128, GDN, 512-slot pool)
runs in full with sampled (sequence, head) pairs recomputed by the oracle."""
import numpy as np
import pytest
import torch

import gated_delta_rule_44_amd as gdr
import oracle
from gated_delta_rule_44_amd import synthetic
from tests.conftest import gpu_available
from tests.gpu_util import announce, assert_close, to_np

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]
DEV = torch.device("cuda:0")
DTYPES = {"fp32": torch.float32, "bf16": torch.bfloat16}
NAMES = ("q", "k", "v", "g", "beta")
SENTINEL = 7.0


def sync():
    torch.cuda.synchronize(DEV)


def _committed(pool0, ck, slot, accepted):
    """The pool after keeping the accepted prefixes, by indexing."""
    want = pool0.clone()
    n = ck.shape[1]
    for b, (s, m) in enumerate(zip(slot, accepted)):
        if 0 <= s < pool0.shape[0] and 1 <= m <= n:
            want[s] = ck[b, m - 1]
    return want


@pytest.mark.parametrize("dt", ["fp32", "bf16"])
@pytest.mark.parametrize("gate", ["scalar", "channel"])
@pytest.mark.parametrize("D", [64, 128])
def test_decode_tokens_checkpoints_commit(dt, gate, D):
    announce("decode_tokens %s %s D=%d" % (dt, gate, D))
    B, n, H, P = 5, 4, 3, 8
    x = synthetic.prefill_inputs(B, n, H, D, DTYPES[dt], gate, seed=31, h0=False, device=DEV)
    pool0 = synthetic.pool_states(P, H, D, seed=32, device=DEV)
    slot_np = synthetic.serving_slots(B, P, idle=1, seed=33)
    slot = torch.from_numpy(slot_np).to(DEV)
    act = np.flatnonzero(slot_np >= 0)
    idle = np.flatnonzero(slot_np < 0)
    unused = np.setdiff1d(np.arange(P), slot_np[act])
    args = [x[k] for k in NAMES]

    # checkpointed: the pool keeps its bytes, the states after each token go out
    pool = pool0.clone()
    o = torch.full_like(x["v"], SENTINEL)
    ck = torch.full((B, n, H, D, D), SENTINEL, device=DEV)
    gdr.decode_tokens(*args, pool, slot=slot, checkpoints=ck, scale=0.8,
                      slot_host=slot_np, o=o)
    sync()
    o_ref, _, ck_ref = oracle.decode_tokens(*args, pool0, slot=slot_np, checkpoints=True,
                                            scale=0.8)
    assert torch.equal(pool, pool0), "checkpointed call changed the pool"
    eo = assert_close(o[act], o_ref[act], DTYPES[dt], "o")
    ec = assert_close(ck[act], ck_ref[act], DTYPES[dt], "checkpoints")
    assert bool((o[idle] == SENTINEL).all()) and bool((ck[idle] == SENTINEL).all()), \
        "idle sequence written"
    assert np.abs(to_np(ck[act]) - ck_ref[act]).max() < 1e-5

    # in place: the pool advances by n tokens, same outputs bit for bit
    o2 = torch.full_like(x["v"], SENTINEL)
    gdr.decode_tokens(*args, pool, slot=slot, scale=0.8, o=o2)
    sync()
    _, pool_ref, _ = oracle.decode_tokens(*args, pool0, slot=slot_np, scale=0.8)
    es = assert_close(pool[slot_np[act]], pool_ref[slot_np[act]], DTYPES[dt], "pool")
    assert torch.equal(pool[unused], pool0[unused]), "unused slot changed"
    assert torch.equal(o2, o), "in-place and checkpointed outputs differ"
    assert torch.equal(pool[slot_np[act]], ck[act, n - 1]), "last checkpoint != pool"

    # commit the accepted prefixes: an exact copy of the chosen checkpoints
    accepted = synthetic.accepted_counts(B, n, seed=34)
    accepted[act[0]] = 0                  # a fully rejected draft keeps its state
    accepted[act[1]] = n
    pool3 = pool0.clone()
    gdr.decode_commit(ck, torch.from_numpy(accepted).to(DEV), pool3, slot=slot)
    sync()
    assert torch.equal(pool3, _committed(pool0, ck, slot_np, accepted)), "commit"
    announce("  err o=%.2e ckpt=%.2e pool=%.2e" % (eo, ec, es))


@pytest.mark.parametrize("dt", ["fp32", "bf16"])
@pytest.mark.parametrize("gate", ["scalar", "channel"])
def test_decode_tokens_one_token_is_decode_step(dt, gate):
    announce("decode_tokens n=1 vs decode_step %s %s" % (dt, gate))
    B, H, D = 6, 4, 128
    x = synthetic.prefill_inputs(B, 1, H, D, DTYPES[dt], gate, seed=35, device=DEV)
    st = x["h0"].clone()
    o1 = gdr.decode_step(*[x[k][:, 0].contiguous() for k in NAMES], st, scale=0.6)
    pool = x["h0"].clone()
    o2 = gdr.decode_tokens(*[x[k] for k in NAMES], pool, scale=0.6)
    sync()
    # the same fp32 update in another kernel: equal up to the compiler's
    # choice of fused multiply-adds
    assert (pool - st).abs().max().item() < 1e-6
    tol = 1e-6 if dt == "fp32" else 2.0 ** -8      # one bf16 rounding step
    assert ((o2[:, 0].float() - o1.float()).abs() <= tol * o1.float().abs() + 1e-6).all()


@pytest.mark.parametrize("gate", ["scalar", "channel"])
def test_decode_tokens_long_draft(gate):
    announce("decode_tokens n=24 bf16 %s" % gate)
    B, n, H, D, P = 3, 24, 2, 128, 4
    x = synthetic.prefill_inputs(B, n, H, D, torch.bfloat16, gate, seed=36, h0=False,
                                 device=DEV)
    pool0 = synthetic.pool_states(P, H, D, seed=37, device=DEV)
    slot_np = np.array([3, 0, 2], np.int32)
    pool = pool0.clone()
    o, ck = gdr.decode_tokens(*[x[k] for k in NAMES], pool, slot=torch.from_numpy(slot_np).to(DEV),
                              checkpoints=True)
    sync()
    o_ref, _, ck_ref = oracle.decode_tokens(*[x[k] for k in NAMES], pool0, slot=slot_np,
                                            checkpoints=True)
    assert_close(o, o_ref, torch.bfloat16, "o")
    assert_close(ck, ck_ref, torch.bfloat16, "checkpoints")


def test_decode_tokens_all_idle_writes_nothing():
    announce("decode_tokens all idle")
    B, n, H, D, P = 4, 3, 2, 64, 3
    x = synthetic.prefill_inputs(B, n, H, D, torch.bfloat16, "channel", seed=38, h0=False,
                                 device=DEV)
    pool0 = synthetic.pool_states(P, H, D, seed=39, device=DEV)
    pool = pool0.clone()
    o = torch.full_like(x["v"], SENTINEL)
    slot = torch.tensor([-1, 3, -7, 1 << 20], dtype=torch.int32, device=DEV)  # all out of range
    gdr.decode_tokens(*[x[k] for k in NAMES], pool, slot=slot, o=o)
    sync()
    assert torch.equal(pool, pool0) and bool((o == SENTINEL).all())


@pytest.mark.parametrize("dt", ["fp32", "bf16"])
@pytest.mark.parametrize("gate", ["scalar", "channel"])
@pytest.mark.parametrize("D", [64, 128])
def test_prefill_varlen_pool(dt, gate, D):
    announce("prefill_varlen_pool %s %s D=%d" % (dt, gate, D))
    lens = [70, 0, 130, 33, 64]
    H, P = 3, 7
    x = synthetic.varlen_inputs(lens, H, D, DTYPES[dt], gate, seed=40, h0=False, device=DEV)
    pool0 = synthetic.pool_states(P, H, D, seed=41, device=DEV)
    h0_np = np.array([2, 0, -1, 5, 6], np.int32)       # 2: in place; -1: from zeros
    ht_np = np.array([2, 4, 1, -1, 3], np.int32)       # -1: not stored
    pool = pool0.clone()
    o = gdr.prefill_varlen_pool(*[x[k] for k in NAMES], x["cu_seqlens"], pool,
                                torch.from_numpy(h0_np).to(DEV), torch.from_numpy(ht_np).to(DEV),
                                scale=0.9, cu_seqlens_host=x["cu_seqlens_host"],
                                slots_host=(h0_np, ht_np))
    sync()
    o_ref, pool_ref = oracle.forward_pool(*[x[k] for k in NAMES], x["cu_seqlens_host"],
                                          pool0, h0_np, ht_np, scale=0.9)
    eo = assert_close(o, o_ref, DTYPES[dt], "o")
    written = ht_np[ht_np >= 0]
    es = assert_close(pool[written], pool_ref[written], DTYPES[dt], "pool")
    kept = np.setdiff1d(np.arange(P), written)
    assert torch.equal(pool[kept], pool0[kept]), "slot not written by any sequence changed"
    # the empty sequence copies its start state exactly
    assert torch.equal(pool[4], pool0[0])
    announce("  err o=%.2e pool=%.2e" % (eo, es))


def test_draft_decode_workload_B256_n4_H32():
    """Drafted decode at full size: GDN, bf16, 4 tokens, a 512-slot pool."""
    announce("workload gdn_draft_decode_B256_n4_H32_d128_bf16")
    B, n, H, D, P = 256, 4, 32, 128, 512
    x = synthetic.prefill_inputs(B, n, H, D, torch.bfloat16, "scalar", seed=1005,
                                 h0=False, device=DEV)
    pool = synthetic.pool_states(P, H, D, seed=1006, device=DEV)
    slot_np = synthetic.serving_slots(B, P, idle=0, seed=1007)
    slot = torch.from_numpy(slot_np).to(DEV)
    accepted = synthetic.accepted_counts(B, n, seed=1008)
    rng = np.random.default_rng(5)
    samples = [(int(rng.integers(B)), int(rng.integers(H))) for _ in range(24)]
    before = {s: pool[slot_np[s[0]], s[1]].clone() for s in samples}
    o, ck = gdr.decode_tokens(*[x[k] for k in NAMES], pool, slot=slot, checkpoints=True)
    gdr.decode_commit(ck, torch.from_numpy(accepted).to(DEV), pool, slot=slot)
    sync()
    assert bool(torch.isfinite(o).all())
    got, ref = {"o": [], "ck": [], "pool": []}, {"o": [], "ck": [], "pool": []}
    for (b, h) in samples:
        sl = [x[k][b:b + 1, :, h:h + 1].contiguous() for k in NAMES]
        oo, _, cc = oracle.decode_tokens(*sl, before[(b, h)][None, None], checkpoints=True)
        got["o"].append(to_np(o[b, :, h]))
        ref["o"].append(oo[0, :, 0])
        got["ck"].append(to_np(ck[b, :, h]))
        ref["ck"].append(cc[0, :, 0])
        m = int(accepted[b])
        got["pool"].append(to_np(pool[slot_np[b], h]))
        ref["pool"].append(cc[0, m - 1, 0] if m >= 1 else to_np(before[(b, h)]))
    errs = [assert_close(np.stack(got[k]), np.stack(ref[k]), torch.bfloat16, k)
            for k in ("o", "ck", "pool")]
    announce("  24 sampled pairs: rel-fro o=%.2e ckpt=%.2e committed=%.2e" % tuple(errs))


def test_kda_varlen_pool_workload_matches_plain_varlen():
    """The KDA packed workload (16 sequences, 300,686 tokens, H=32) through a
    pool is the plain packed call with the gathered start states: the same
    kernels, so the same bits."""
    announce("workload kda_varlen_N16_H32 through a 40-slot pool")
    lens = synthetic.varlen_lengths(943)
    N, H, D, P = len(lens), 32, 128, 40
    x = synthetic.varlen_inputs(lens, H, D, torch.bfloat16, "channel", seed=1004,
                                h0=False, device=DEV)
    pool = synthetic.pool_states(P, H, D, seed=1009, device=DEV)
    h0_np = synthetic.serving_slots(N, P, idle=2, seed=1010)
    ht_np = np.array([s for s in range(P) if s not in set(h0_np.tolist())][:N], np.int32)
    h0 = torch.zeros((N, H, D, D), device=DEV)
    for i, s in enumerate(h0_np):
        if s >= 0:
            h0[i] = pool[s]
    o_ref, ht_ref = gdr.prefill_varlen(*[x[k] for k in NAMES], x["cu_seqlens"], h0=h0,
                                       cu_seqlens_host=x["cu_seqlens_host"])
    keep = pool.clone()
    o = gdr.prefill_varlen_pool(*[x[k] for k in NAMES], x["cu_seqlens"], pool,
                                torch.from_numpy(h0_np).to(DEV), torch.from_numpy(ht_np).to(DEV),
                                cu_seqlens_host=x["cu_seqlens_host"], slots_host=(h0_np, ht_np))
    sync()
    assert torch.equal(o, o_ref)
    assert torch.equal(pool[ht_np], ht_ref)
    rest = np.setdiff1d(np.arange(P), ht_np)
    assert torch.equal(pool[rest], keep[rest])
