"""GPU parity of the chunked prefill over the whole range of the gate.

The recurrence takes any gate a in [0, 1], that is any g = ln a in
[-inf, 0], per head (GDN) or per key channel (KDA) ("Super Apriel: One
Checkpoint, Many Speeds", gist.science summary 2a, for the two gate kinds).
The chunked form factors the in-chunk decay e^{b_r - b_s}; these cases push
it where a naive factorisation e^{b_r} e^{-b_s} overflows or meets
-inf - (-inf): gates of exactly zero (g = -inf) at a chunk start, in the
middle of a chunk and in a ragged tail, a constant g = -4 per token (-256
per chunk), per-channel mixtures of -inf and -0.01, and single 16-token
blocks that decay by more than e^70 in some channels.  Every output must be
finite and meet the bf16 bar against the fp64 oracle, which takes a = e^g
token by token and has no range limit."""
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
NEG_INF = float("-inf")
# token positions of a T = 200 sequence: chunk starts (0, 64), the middle of
# a chunk (100), the last row of a 16-token block (143) and the ragged tail
# (chunk 3 holds tokens 192..199)
ZERO_AT = [0, 64, 100, 143, 195]


def sync():
    torch.cuda.synchronize(DEV)


def gate_pattern(name, g, gate, seed=0):
    """The gate logs g (a CPU or device tensor [.., T, H(, D)]) overwritten
    with one of the test patterns; token axis 1 for [B, T, ...]."""
    g = g.clone()
    rng = np.random.default_rng(seed)
    if name == "zero_tokens":
        for t in ZERO_AT:
            if t < g.shape[1]:
                g[:, t] = NEG_INF
    elif name == "const4":
        g.fill_(-4.0)
    elif name == "mix_inf":
        m = torch.from_numpy(rng.random(tuple(g.shape)) < 0.05).to(g.device)
        g = torch.where(m, torch.full_like(g, NEG_INF), torch.full_like(g, -0.01))
    elif name == "block_decay":
        # a few channels (KDA) or every head (GDN) decay by e^-6 per token:
        # a 16-token block loses e^-96, beyond e^70
        if gate == "channel":
            g[..., :8] = -6.0
            g[..., 64:66] = -100.0
        else:
            g.fill_(-6.0)
    elif name == "strong":
        g = g * 100.0                       # -softplus(N) * 10 (GDN) / 5 (KDA)
    else:
        raise ValueError(name)
    return g.contiguous()


PATTERNS = ["zero_tokens", "const4", "mix_inf", "block_decay", "strong"]


def check(x, o, ht, what):
    assert bool(torch.isfinite(o.float()).all()), "%s: o not finite" % what
    assert bool(torch.isfinite(ht).all()), "%s: ht not finite" % what
    o_ref, ht_ref = oracle.forward(x["q"], x["k"], x["v"], x["g"], x["beta"], h0=x["h0"],
                                   cu_seqlens=x.get("cu_seqlens_host"))
    eo = assert_close(o, o_ref, torch.bfloat16, what + " o")
    eh = assert_close(ht, ht_ref, torch.bfloat16, what + " ht")
    announce("  %s: rel-fro o=%.2e ht=%.2e" % (what, eo, eh))


@pytest.mark.parametrize("gate", ["scalar", "channel"])
@pytest.mark.parametrize("pattern", PATTERNS)
@pytest.mark.parametrize("D", [64, 128])
def test_prefill_gate_range(gate, pattern, D):
    announce("gate range %s %s D=%d" % (gate, pattern, D))
    x = synthetic.prefill_inputs(2, 200, 3, D, torch.bfloat16, gate, seed=80, device=DEV)
    x["g"] = gate_pattern(pattern, x["g"], gate, seed=81)
    o, ht = gdr.prefill(x["q"], x["k"], x["v"], x["g"], x["beta"], h0=x["h0"])
    sync()
    check(x, o, ht, "%s %s" % (gate, pattern))


@pytest.mark.parametrize("gate", ["scalar", "channel"])
def test_prefill_gate_zero_everywhere(gate):
    """a = 0 on every token: each state is beta v k^T of its own token, and
    o_t = beta_t v_t (k_t.q_t)."""
    announce("gate zero everywhere %s" % gate)
    x = synthetic.prefill_inputs(1, 150, 2, 128, torch.bfloat16, gate, seed=82, device=DEV)
    x["g"] = torch.full_like(x["g"], NEG_INF)
    o, ht = gdr.prefill(x["q"], x["k"], x["v"], x["g"], x["beta"], h0=x["h0"])
    sync()
    check(x, o, ht, "%s all zero" % gate)


@pytest.mark.parametrize("gate", ["scalar", "channel"])
@pytest.mark.parametrize("pattern", ["zero_tokens", "mix_inf", "block_decay"])
def test_prefill_varlen_gate_range(gate, pattern):
    lens = [200, 0, 1, 64, 130, 17]
    announce("varlen gate range %s %s" % (gate, pattern))
    x = synthetic.varlen_inputs(lens, 2, 128, torch.bfloat16, gate, seed=83, device=DEV)
    g = gate_pattern(pattern, x["g"][None], gate, seed=84)[0]
    x["g"] = g.contiguous()
    o, ht = gdr.prefill_varlen(x["q"], x["k"], x["v"], x["g"], x["beta"], x["cu_seqlens"],
                               h0=x["h0"], cu_seqlens_host=x["cu_seqlens_host"])
    sync()
    check(x, o, ht, "varlen %s %s" % (gate, pattern))


@pytest.mark.parametrize("gate", ["scalar", "channel"])
def test_prefill_fused_gate_range(gate):
    """Raw gate logits that make g = -c softplus(x) huge or -inf (a bf16
    logit of +inf), on the fused-preprocessing path."""
    announce("fused gate range %s" % gate)
    x = synthetic.raw_prefill_inputs(2, 200, 2, 128, torch.bfloat16, gate, seed=85, device=DEV)
    xg = x["gate_logit"].float()
    xg[:, 64] = float("inf")
    xg[:, 100:118] = 300.0
    xg[:, 195] = 1e4
    x["gate_logit"] = xg.to(torch.bfloat16).contiguous()
    raw = ("q", "k", "v", "gate_logit", "beta_logit")
    o, ht = gdr.prefill_fused(*[x[n] for n in raw], x["gate_scale"], h0=x["h0"])
    sync()
    qh, kh, g, beta = oracle.preprocess(x["q"], x["k"], x["gate_logit"], x["beta_logit"],
                                        x["gate_scale"])
    assert np.isneginf(g).any()
    assert bool(torch.isfinite(o.float()).all()) and bool(torch.isfinite(ht).all())
    o_ref, ht_ref = oracle.forward(qh, kh, x["v"], g, beta, h0=x["h0"])
    eo = assert_close(o, o_ref, torch.bfloat16, "o")
    eh = assert_close(ht, ht_ref, torch.bfloat16, "ht")
    announce("  rel-fro o=%.2e ht=%.2e" % (eo, eh))


@pytest.mark.parametrize("dt", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("gate", ["scalar", "channel"])
def test_recurrent_and_decode_gate_range(dt, gate):
    """The token-by-token forms (fp32 prefill, decode) take a = e^g as is."""
    announce("recurrent/decode gate range %s %s" % (dt, gate))
    x = synthetic.prefill_inputs(2, 70, 2, 64, dt, gate, seed=86, device=DEV)
    x["g"] = gate_pattern("mix_inf", x["g"], gate, seed=87)
    if dt == torch.float32:
        o, ht = gdr.prefill(x["q"], x["k"], x["v"], x["g"], x["beta"], h0=x["h0"])
        sync()
        o_ref, ht_ref = oracle.forward(x["q"], x["k"], x["v"], x["g"], x["beta"], h0=x["h0"])
        assert_close(o, o_ref, dt, "o")
        assert_close(ht, ht_ref, dt, "ht")
    one = {n: x[n][:, 5].contiguous() for n in ("q", "k", "v", "g", "beta")}
    st = x["h0"].clone()
    od = gdr.decode_step(one["q"], one["k"], one["v"], one["g"], one["beta"], st)
    sync()
    od_ref, st_ref = oracle.decode(one["q"], one["k"], one["v"], one["g"], one["beta"], x["h0"])
    assert_close(od, od_ref, dt, "decode o")
    assert_close(st, st_ref, dt, "decode state")
