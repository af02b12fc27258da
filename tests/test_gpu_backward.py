"""GPU parity of the backward (gdr_backward_chunked) against the fp64
oracle: oracle.backward differentiates a token-by-token fp64 forward by
autograd (pinned on the CPU by finite differences).  Every gradient --
dq, dk, dv, dg, dbeta, dh0 -- is compared over the whole tensor with the
bf16 bar, at sizes that span several chunks and a ragged tail, and at the
prefill workloads' full sizes on sampled (sequence, head) pairs."""
import numpy as np
import pytest
import torch

import gated_delta_rule_44_amd as gdr
import oracle
from gated_delta_rule_44_amd import synthetic
from tests.conftest import gpu_available
from tests.gpu_util import announce, assert_close

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]
DEV = torch.device("cuda:0")
NAMES = ("dq", "dk", "dv", "dg", "dbeta", "dh0")


def sync():
    torch.cuda.synchronize(DEV)


def _upstream(B, T, H, D, seed):
    gen = torch.Generator(device=DEV)
    gen.manual_seed(seed)
    do = torch.randn((B, T, H, D), generator=gen, device=DEV).to(torch.bfloat16)
    dht = torch.randn((B, H, D, D), generator=gen, device=DEV) * 0.1
    return do, dht


def _check(got, ref, what):
    errs = []
    for n, x, r in zip(NAMES, got, ref):
        errs.append(assert_close(x, r, torch.bfloat16, "%s %s" % (what, n)))
    announce("  rel-fro " + " ".join("%s=%.1e" % (n, e) for n, e in zip(NAMES, errs)))


@pytest.mark.parametrize("gate", ["scalar", "channel"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("T", [1, 64, 65, 150])
def test_backward(gate, D, T):
    announce("backward %s D=%d T=%d" % (gate, D, T))
    B, H = 2, 2
    x = synthetic.prefill_inputs(B, T, H, D, torch.bfloat16, gate, seed=70 + T, device=DEV)
    do, dht = _upstream(B, T, H, D, 80 + T)
    got = gdr.backward(x["q"], x["k"], x["v"], x["g"], x["beta"], do, h0=x["h0"], dht=dht,
                       scale=0.8)
    sync()
    ref = oracle.backward(x["q"], x["k"], x["v"], x["g"], x["beta"], do, h0=x["h0"], dht=dht,
                          scale=0.8)
    _check(got, ref, "%s D=%d T=%d" % (gate, D, T))


@pytest.mark.parametrize("gate", ["scalar", "channel"])
def test_backward_strong_decay(gate):
    """Gates of about -50 per 64 tokens (the forward's strong-decay case):
    the chunk's e^{+-b} factors span ~20 orders of magnitude, in the gated
    operands and in dq = dQt e^b, dk = dKt e^b + dKb e^-b."""
    B, T, H, D = 1, 150, 2, 128
    x = synthetic.prefill_inputs(B, T, H, D, torch.bfloat16, gate, seed=21, device=DEV,
                                 gate_scale=1.0)
    announce("backward strong decay %s: min gate sum over the first chunk %.1f"
             % (gate, float(x["g"][0, :64].sum(0).min())))
    do, dht = _upstream(B, T, H, D, 90)
    got = gdr.backward(x["q"], x["k"], x["v"], x["g"], x["beta"], do, h0=x["h0"], dht=dht)
    sync()
    ref = oracle.backward(x["q"], x["k"], x["v"], x["g"], x["beta"], do, h0=x["h0"], dht=dht)
    _check(got, ref, "strong decay %s" % gate)


@pytest.mark.parametrize("gate", ["scalar", "channel"])
def test_backward_without_h0_and_dht(gate):
    announce("backward no h0/dht %s" % gate)
    B, T, H, D = 1, 100, 3, 128
    x = synthetic.prefill_inputs(B, T, H, D, torch.bfloat16, gate, seed=90, h0=False, device=DEV)
    do, _ = _upstream(B, T, H, D, 91)
    got = gdr.backward(x["q"], x["k"], x["v"], x["g"], x["beta"], do)
    sync()
    ref = oracle.backward(x["q"], x["k"], x["v"], x["g"], x["beta"], do)
    _check(got, ref, gate)


def test_backward_empty_sequence():
    announce("backward T=0")
    x = synthetic.prefill_inputs(2, 0, 2, 128, torch.bfloat16, "channel", seed=92, device=DEV)
    do, dht = _upstream(2, 0, 2, 128, 93)
    got = gdr.backward(x["q"], x["k"], x["v"], x["g"], x["beta"], do, h0=x["h0"], dht=dht)
    sync()
    assert torch.equal(got[5], dht)
    got = gdr.backward(x["q"], x["k"], x["v"], x["g"], x["beta"], do, h0=x["h0"])
    sync()
    assert bool((got[5] == 0).all())


def _sampled(B, T, H, gate, seed, pairs):
    x = synthetic.prefill_inputs(B, T, H, 128, torch.bfloat16, gate, seed=seed,
                                 h0=gate == "scalar", device=DEV)
    do, dht = _upstream(B, T, H, 128, seed + 50)
    got = gdr.backward(x["q"], x["k"], x["v"], x["g"], x["beta"], do, h0=x["h0"], dht=dht)
    sync()
    for t in got:
        assert bool(torch.isfinite(t).all())
    for b, h in pairs:
        sl = lambda t: t[b:b + 1, :, h:h + 1].contiguous()  # noqa: E731
        h0 = None if x["h0"] is None else x["h0"][b:b + 1, h:h + 1].contiguous()
        ref = oracle.backward(sl(x["q"]), sl(x["k"]), sl(x["v"]), sl(x["g"]), sl(x["beta"]),
                              sl(do), h0=h0, dht=dht[b:b + 1, h:h + 1].contiguous())
        mine = [sl(t) for t in got[:5]] + [got[5][b:b + 1, h:h + 1]]
        _check(mine, ref, "(b=%d, h=%d)" % (b, h))


def test_backward_gdn_B4_H16_T4096():
    announce("backward GDN B=4 H=16 T=4096")
    _sampled(4, 4096, 16, "scalar", 1001, [(0, 0), (3, 15)])


def test_backward_kda_B2_H32_T8192():
    announce("backward KDA B=2 H=32 T=8192")
    _sampled(2, 8192, 32, "channel", 1002, [(1, 7)])
