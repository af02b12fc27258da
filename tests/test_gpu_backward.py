"""GPU parity of the backward (gdr_backward_chunked) against the fp64
oracle: oracle.backward differentiates a token-by-token fp64 forward by
autograd (pinned on the CPU by finite differences).  Every gradient --
dq, dk, dv, dg, dbeta, dh0 -- is compared over the whole tensor with the
bf16 bar, at sizes that span several chunks and a ragged tail, and at the
prefill workloads' full sizes on every (sequence, head) against the C
oracle's fp64 backward (oracle.backward_c, pinned to the autograd form).
Gates past the chunk factorisation's range go through the token-level
path and are checked here too."""
import numpy as np
import pytest
import torch

import gated_delta_rule_44_amd as gdr
import oracle
from gated_delta_rule_44_amd import synthetic
from tests.conftest import gpu_available
from tests.gpu_util import announce, assert_close, heads_first, to_np

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


def _gate_pattern(x, pattern):
    """Gates past the chunk factorisation's range (a chunk decaying by more
    than e^80 in some channel), written into x["g"] ([B, T, H(, D)])."""
    g = x["g"]
    if pattern == "mixed":
        g[0, 64:90, 1] = -6.0                  # pair (0, 1): chunk 1 decays by e^-156
        g[1, 10, 0] = float("-inf")            # pair (1, 0): one zero gate, in range
    elif pattern == "constant":
        g.fill_(-4.0)                          # every chunk of every pair: e^-256
    elif pattern == "zeros":
        for t in (64, 100, 149):               # a = 0 at a chunk start, mid-chunk, in the tail
            g[:, t] = float("-inf")
        g[0, 20:40, 0] = -5.0                  # and one pair past the range
    elif pattern == "channel_mix":
        if g.dim() == 4:                       # -inf and -0.01 in alternate channels
            g[:, 30:50, :, 0::2] = float("-inf")
            g[:, 30:50, :, 1::2] = -0.01
        else:
            g[:, 30:50] = float("-inf")
    return x


@pytest.mark.parametrize("pattern", ["mixed", "constant", "zeros", "channel_mix"])
@pytest.mark.parametrize("gate", ["scalar", "channel"])
@pytest.mark.parametrize("D", [64, 128])
def test_backward_beyond_the_chunk_range(gate, D, pattern):
    """The chunk-local gradients factor each chunk from its first token,
    which holds while no channel decays by more than e^80 over a chunk; the
    pairs where one does are recomputed by the token-level adjoint.  Every
    pair is compared with the oracle (gates of zero included, which the
    kernels raise to -30 like the forward), and a second call gives the same
    bits (dg and dbeta to fp32 rounding: the in-range pairs sum them in
    whatever order LDS float atomics arrive)."""
    announce("backward beyond the chunk range %s D=%d %s" % (gate, D, pattern))
    B, T, H = 2, 150, 2
    x = _gate_pattern(synthetic.prefill_inputs(B, T, H, D, torch.bfloat16, gate, seed=73,
                                               device=DEV), pattern)
    do, dht = _upstream(B, T, H, D, 74)
    got = gdr.backward(x["q"], x["k"], x["v"], x["g"], x["beta"], do, h0=x["h0"], dht=dht,
                       scale=0.8)
    again = gdr.backward(x["q"], x["k"], x["v"], x["g"], x["beta"], do, h0=x["h0"], dht=dht,
                         scale=0.8)
    sync()
    for n, t1, t2 in zip(NAMES, got, again):
        if n in ("dg", "dbeta"):   # the in-range pairs sum these with LDS float atomics
            assert float((t1 - t2).abs().max()) <= 1e-5 * float(t1.abs().max()), n
        else:
            assert torch.equal(t1, t2), "%s differs between two calls" % n
    ref = oracle.backward(x["q"], x["k"], x["v"], x["g"], x["beta"], do, h0=x["h0"], dht=dht,
                          scale=0.8)
    for b in range(B):
        for h in range(H):
            mine = [t[b:b + 1, :, h:h + 1] for t in got[:5]] + [got[5][b:b + 1, h:h + 1]]
            rf = [r[b:b + 1, :, h:h + 1] for r in ref[:5]] + [ref[5][b:b + 1, h:h + 1]]
            _check(mine, rf, "%s %s (b=%d, h=%d)" % (gate, pattern, b, h))


def _varlen_case(lens, H, D, gate, seed, scale=0.8):
    x = synthetic.varlen_inputs(lens, H, D, torch.bfloat16, gate, seed=seed, device=DEV)
    cu = x["cu_seqlens_host"]
    Tt, N = int(cu[-1]), len(lens)
    gen = torch.Generator(device=DEV)
    gen.manual_seed(seed + 1)
    do = torch.randn((Tt, H, D), generator=gen, device=DEV).to(torch.bfloat16)
    dht = torch.randn((N, H, D, D), generator=gen, device=DEV) * 0.1
    return x, do, dht


def _varlen_oracle(x, do, dht, scale):
    """oracle.backward sequence by sequence (an empty sequence: dh0 = dht)."""
    cu = x["cu_seqlens_host"]
    N = len(cu) - 1
    Tt, H, D = x["q"].shape
    ref = [np.zeros((Tt, H, D)), np.zeros((Tt, H, D)), np.zeros((Tt, H, D)),
           np.zeros(tuple(x["g"].shape)), np.zeros((Tt, H)), np.zeros((N, H, D, D))]
    for n in range(N):
        a, b = int(cu[n]), int(cu[n + 1])
        if b == a:
            ref[5][n] = dht[n].double().cpu().numpy()
            continue
        r = oracle.backward(*(t[a:b][None] for t in (x["q"], x["k"], x["v"], x["g"],
                                                      x["beta"], do)),
                            h0=x["h0"][n:n + 1], dht=dht[n:n + 1], scale=scale)
        for i in range(5):
            ref[i][a:b] = r[i][0]
        ref[5][n] = r[5][0]
    return ref


@pytest.mark.parametrize("gate", ["scalar", "channel"])
@pytest.mark.parametrize("D", [64, 128])
def test_backward_varlen(gate, D):
    """A packed batch with ragged tails, a one-token and an empty sequence."""
    lens = [150, 1, 0, 64, 65, 200]
    announce("backward varlen %s D=%d lengths %s" % (gate, D, lens))
    x, do, dht = _varlen_case(lens, 2, D, gate, 60 + D)
    got = gdr.backward_varlen(x["q"], x["k"], x["v"], x["g"], x["beta"], do, x["cu_seqlens"],
                              h0=x["h0"], dht=dht, scale=0.8,
                              cu_seqlens_host=x["cu_seqlens_host"])
    sync()
    _check(got, _varlen_oracle(x, do, dht, 0.8), "varlen %s D=%d" % (gate, D))


@pytest.mark.parametrize("gate", ["scalar", "channel"])
def test_backward_varlen_beyond_the_chunk_range(gate):
    """A packed batch where some sequences decay by more than e^80 over a
    chunk (one of them with a zero gate in its ragged tail) next to ones in
    range."""
    lens = [150, 1, 0, 64, 65, 200]
    announce("backward varlen beyond the chunk range %s lengths %s" % (gate, lens))
    x, do, dht = _varlen_case(lens, 2, 128, gate, 64)
    cu = x["cu_seqlens_host"]
    g = x["g"]
    g[int(cu[0]):int(cu[1])] = -4.0            # sequence 0, both heads
    g[int(cu[5]) + 70:int(cu[5]) + 100, 1] = -5.0   # sequence 5, head 1
    g[int(cu[5]) + 190, 1] = float("-inf")
    g[int(cu[4]) + 64, 0] = float("-inf")      # sequence 4: a zero gate, in range
    got = gdr.backward_varlen(x["q"], x["k"], x["v"], x["g"], x["beta"], do, x["cu_seqlens"],
                              h0=x["h0"], dht=dht, scale=0.8,
                              cu_seqlens_host=x["cu_seqlens_host"])
    sync()
    _check(got, _varlen_oracle(x, do, dht, 0.8), "varlen beyond the range %s" % gate)


def test_backward_varlen_long_sequences():
    """Sequences of 700 to 3000 tokens, channel gate, d = 128."""
    lens = [700, 3000, 17, 640]
    announce("backward varlen channel D=128 lengths %s" % lens)
    x, do, dht = _varlen_case(lens, 2, 128, "channel", 77)
    got = gdr.backward_varlen(x["q"], x["k"], x["v"], x["g"], x["beta"], do, x["cu_seqlens"],
                              h0=x["h0"], dht=dht, scale=0.8)
    sync()
    _check(got, _varlen_oracle(x, do, dht, 0.8), "varlen long")


@pytest.mark.parametrize("gate", ["scalar", "channel"])
def test_backward_varlen_equal_lengths_match_fixed(gate):
    """A packed batch of equal lengths is the fixed-length batch: the same
    kernels on the same chunks give the same bits -- except where LDS float
    atomics sum a chunk's rows in whatever order they arrive (dg, dbeta),
    which agree to fp32 rounding."""
    B, T, H, D = 3, 150, 2, 128
    x = synthetic.prefill_inputs(B, T, H, D, torch.bfloat16, gate, seed=88, device=DEV)
    do, dht = _upstream(B, T, H, D, 89)
    fixed = gdr.backward(x["q"], x["k"], x["v"], x["g"], x["beta"], do, h0=x["h0"], dht=dht)
    cu = torch.arange(0, (B + 1) * T, T, dtype=torch.int32, device=DEV)
    flat = lambda t: t.reshape((B * T,) + tuple(t.shape[2:]))  # noqa: E731
    packed = gdr.backward_varlen(*(flat(x[n]) for n in ("q", "k", "v", "g", "beta")), flat(do),
                                 cu, h0=x["h0"], dht=dht)
    sync()
    for n, a, b in zip(NAMES, fixed, packed):
        a = a if n == "dh0" else flat(a)
        if n in ("dg", "dbeta"):
            assert float((a - b).abs().max()) <= 1e-5 * float(a.abs().max()), n
        else:
            assert torch.equal(a, b), n


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


def _every_pair(B, T, H, gate, seed):
    """The backward at a workload's full size against the C oracle's fp64
    backward, each (sequence, head) on its own with the bf16 bar (and every
    token row within the row bar)."""
    x = synthetic.prefill_inputs(B, T, H, 128, torch.bfloat16, gate, seed=seed,
                                 h0=gate == "scalar", device=DEV)
    do, dht = _upstream(B, T, H, 128, seed + 50)
    got = gdr.backward(x["q"], x["k"], x["v"], x["g"], x["beta"], do, h0=x["h0"], dht=dht)
    sync()
    got = [to_np(t) for t in got]
    for t in got:
        assert np.all(np.isfinite(t))
    ref = oracle.backward_c(x["q"], x["k"], x["v"], x["g"], x["beta"], do, h0=x["h0"],
                            dht=dht)
    worst = {}
    for n, gt, rf in zip(NAMES, got, ref):
        if n == "dh0":
            gt, rf = gt.reshape(B * H, 128, 128), rf.reshape(B * H, 128, 128)
        else:
            gt, rf = heads_first(gt), heads_first(rf)
        for p in range(B * H):
            e = assert_close(gt[p], rf[p], torch.bfloat16, "%s pair %d" % (n, p))
            worst[n] = max(worst.get(n, 0.0), e)
    announce("  worst pair rel-fro " + " ".join("%s=%.1e" % (n, worst[n]) for n in NAMES))


# every (sequence, head), so that the chunk-to-workgroup mappings of all
# three stages are checked (the C oracle takes a few seconds per workload
# on the host threads)
def test_backward_gdn_B4_H16_T4096():
    announce("backward GDN B=4 H=16 T=4096, every pair")
    _every_pair(4, 4096, 16, "scalar", 1001)


def test_backward_kda_B2_H32_T8192():
    announce("backward KDA B=2 H=32 T=8192, every pair")
    _every_pair(2, 8192, 32, "channel", 1002)
