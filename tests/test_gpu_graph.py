"""HIP graph capture of the library's calls.  Every entry point only
launches kernels on the caller's stream (no allocation, no memset, no
synchronisation), so a call captured once replays on new inputs copied
into the same buffers.  Each graph is replayed several times, with eager
work and synchronisations in between, and every replay is checked against
an eager call on the same inputs."""
import pytest
import torch

import gated_delta_rule_44_amd as gdr
from gated_delta_rule_44_amd import synthetic
from tests.conftest import gpu_available
from tests.gpu_util import announce

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]
DEV = torch.device("cuda:0")


def _capture(fn):
    """Warm up on a side stream, then capture fn() into a graph."""
    side = torch.cuda.Stream(DEV)
    side.wait_stream(torch.cuda.current_stream(DEV))
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream(DEV).wait_stream(side)
    torch.cuda.synchronize(DEV)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        out = fn()
    torch.cuda.synchronize(DEV)
    return graph, out


def _load(dst, src):
    for name, t in dst.items():
        if torch.is_tensor(t):
            t.copy_(src[name])


@pytest.mark.parametrize("gate", ["scalar", "channel"])
def test_prefill_graph_replays(gate):
    B, T, H, D = 2, 200, 2, 128
    x = synthetic.prefill_inputs(B, T, H, D, torch.bfloat16, gate, seed=5, device=DEV)
    ws = torch.empty(gdr.workspace_bytes(torch.bfloat16, gate == "channel", B, B * T, H),
                     device=DEV, dtype=torch.uint8)
    run = lambda: gdr.prefill(x["q"], x["k"], x["v"], x["g"], x["beta"],  # noqa: E731
                              h0=x["h0"], workspace=ws)
    graph, (o, ht) = _capture(run)
    for rep in range(3):
        y = synthetic.prefill_inputs(B, T, H, D, torch.bfloat16, gate, seed=10 + rep, device=DEV)
        _load(x, y)
        graph.replay()
        torch.cuda.synchronize(DEV)
        o_g, ht_g = o.clone(), ht.clone()
        o_e, ht_e = gdr.prefill(y["q"], y["k"], y["v"], y["g"], y["beta"], h0=y["h0"])
        torch.cuda.synchronize(DEV)
        announce("prefill %s replay %d" % (gate, rep))
        assert torch.equal(o_g, o_e) and torch.equal(ht_g, ht_e), rep


@pytest.mark.parametrize("gate", ["scalar", "channel"])
def test_backward_graph_replays(gate):
    B, T, H, D = 2, 150, 2, 128
    x = synthetic.prefill_inputs(B, T, H, D, torch.bfloat16, gate, seed=6, device=DEV)
    x["do"] = torch.zeros((B, T, H, D), device=DEV, dtype=torch.bfloat16)
    x["dht"] = torch.zeros((B, H, D, D), device=DEV)
    run = lambda: gdr.backward(x["q"], x["k"], x["v"], x["g"], x["beta"], x["do"],  # noqa: E731
                               h0=x["h0"], dht=x["dht"])
    graph, grads = _capture(run)
    for rep in range(3):
        y = synthetic.prefill_inputs(B, T, H, D, torch.bfloat16, gate, seed=20 + rep, device=DEV)
        gen = torch.Generator(device=DEV)
        gen.manual_seed(30 + rep)
        y["do"] = torch.randn((B, T, H, D), generator=gen, device=DEV).to(torch.bfloat16)
        y["dht"] = torch.randn((B, H, D, D), generator=gen, device=DEV) * 0.1
        _load(x, y)
        graph.replay()
        torch.cuda.synchronize(DEV)
        got = [t.clone() for t in grads]
        ref = gdr.backward(y["q"], y["k"], y["v"], y["g"], y["beta"], y["do"], h0=y["h0"],
                           dht=y["dht"])
        torch.cuda.synchronize(DEV)
        announce("backward %s replay %d" % (gate, rep))
        for n, a, b in zip(("dq", "dk", "dv", "dg", "dbeta", "dh0"), got, ref):
            if n in ("dg", "dbeta"):   # summed by LDS atomics in arrival order
                assert float((a - b).abs().max()) <= 1e-5 * float(b.abs().max()), (n, rep)
            else:
                assert torch.equal(a, b), (n, rep)


def test_decode_tokens_graph_replays():
    """Drafted decode with checkpoints and the commit, one graph; the pool
    is reset to the same start before every replay and eager run."""
    B, n, H, D, P = 8, 3, 4, 128, 20
    pool0 = synthetic.pool_states(P, H, D, seed=7, device=DEV)
    slot = torch.tensor(synthetic.serving_slots(B, P, seed=7), dtype=torch.int32, device=DEV)
    acc = torch.tensor(synthetic.accepted_counts(B, n, seed=7), dtype=torch.int32, device=DEV)
    acc.clamp_(min=1)

    def draw(seed):
        gen = torch.Generator(device=DEV)
        gen.manual_seed(seed)
        unit = lambda: torch.nn.functional.normalize(  # noqa: E731
            torch.randn((B, n, H, D), generator=gen, device=DEV), dim=-1).to(torch.bfloat16)
        return {"q": unit(), "k": unit(),
                "v": torch.randn((B, n, H, D), generator=gen, device=DEV).to(torch.bfloat16),
                "g": -torch.rand((B, n, H), generator=gen, device=DEV) * 0.1,
                "beta": torch.rand((B, n, H), generator=gen, device=DEV)}
    x = draw(40)
    pool = pool0.clone()

    def run():
        o, ck = gdr.decode_tokens(x["q"], x["k"], x["v"], x["g"], x["beta"], pool, slot=slot,
                                  checkpoints=True)
        gdr.decode_commit(ck, acc, pool, slot=slot)
        return o, ck
    graph, (o, ck) = _capture(run)
    for rep in range(3):
        y = draw(50 + rep)
        _load(x, y)
        pool.copy_(pool0)
        graph.replay()
        torch.cuda.synchronize(DEV)
        o_g, ck_g, pool_g = o.clone(), ck.clone(), pool.clone()
        pool_e = pool0.clone()
        o_e, ck_e = gdr.decode_tokens(y["q"], y["k"], y["v"], y["g"], y["beta"], pool_e,
                                      slot=slot, checkpoints=True)
        gdr.decode_commit(ck_e, acc, pool_e, slot=slot)
        torch.cuda.synchronize(DEV)
        announce("decode_tokens replay %d" % rep)
        assert torch.equal(o_g, o_e) and torch.equal(ck_g, ck_e) and torch.equal(pool_g, pool_e), rep
