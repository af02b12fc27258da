"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle on
seeded inputs, at sizes the oracle finishes in seconds that still span
several chunks, Dv slices and a ragged tail, plus the edge cases."""
import ctypes

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


def sync():
    torch.cuda.synchronize(DEV)


# ----------------------------------------------------------------- decode
@pytest.mark.parametrize("dt", ["fp32", "bf16"])
@pytest.mark.parametrize("gate", ["scalar", "channel"])
@pytest.mark.parametrize("D", [64, 128])
def test_decode_step(dt, gate, D):
    announce("decode_step %s %s D=%d" % (dt, gate, D))
    x = synthetic.prefill_inputs(5, 1, 3, D, DTYPES[dt], gate, seed=11, device=DEV)
    one = {n: x[n][:, 0].contiguous() for n in ("q", "k", "v", "g", "beta")}
    st = x["h0"].clone()
    o = gdr.decode_step(one["q"], one["k"], one["v"], one["g"], one["beta"], st,
                        scale=0.8)
    sync()
    o_ref, st_ref = oracle.decode(one["q"], one["k"], one["v"], one["g"],
                                  one["beta"], x["h0"], scale=0.8)
    assert_close(o, o_ref, DTYPES[dt], "o")
    assert_close(st, st_ref, DTYPES[dt], "state")
    # the state update itself is fp32 either way
    assert np.abs(to_np(st) - st_ref).max() < 1e-5


@pytest.mark.parametrize("dt", ["fp32", "bf16"])
def test_decode_placement_small(dt):
    announce("decode_placement small %s" % dt)
    place = np.array([0, 2, 1, 3, 3, 0, 2, 1], np.uint8)
    x = synthetic.decode_inputs(8, 6, 3, 128, DTYPES[dt], place=place, seed=12,
                                device=DEV)
    pool0 = x["pool"].clone()
    o = torch.full_like(x["v"], 7.0)
    gdr.decode_placement(place, x["q"], x["k"], x["v"], x["g"], x["beta"],
                         x["pool"], o=o)
    sync()
    for layer, code in enumerate(place):
        if code in (synthetic.FA, synthetic.SWA):
            assert torch.equal(x["pool"][layer], pool0[layer]), "state slot touched"
            assert bool((o[layer] == 7.0).all()), "output slot touched"
            continue
        g = x["g"][layer] if code == synthetic.KDA else x["g"][layer][..., 0]
        o_ref, st_ref = oracle.decode(x["q"][layer], x["k"][layer], x["v"][layer],
                                      g, x["beta"][layer], pool0[layer])
        assert_close(o[layer], o_ref, DTYPES[dt], "o layer %d" % layer)
        assert_close(x["pool"][layer], st_ref, DTYPES[dt], "state layer %d" % layer)


# ---------------------------------------------------------------- prefill
def run_prefill(x, scale=1.0):
    o, ht = gdr.prefill(x["q"], x["k"], x["v"], x["g"], x["beta"], h0=x["h0"],
                        scale=scale)
    sync()
    return o, ht


def check_prefill(x, o, ht, dtype, scale=1.0):
    o_ref, ht_ref = oracle.forward(x["q"], x["k"], x["v"], x["g"], x["beta"],
                                   h0=x["h0"], scale=scale)
    eo = assert_close(o, o_ref, dtype, "o")
    eh = assert_close(ht, ht_ref, dtype, "ht")
    return eo, eh


def test_prefill_recurrent_fp32_small_gdn_d64():
    """The fp32 GDN workload: B=H=1, T=64, d=64, zero initial state."""
    announce("prefill fp32 GDN T=64 d=64")
    x = synthetic.prefill_inputs(1, 64, 1, 64, torch.float32, "scalar", seed=1000,
                                 h0=False, device=DEV)
    o, ht = run_prefill(x)
    eo, eh = check_prefill(x, o, ht, torch.float32)
    announce("  max-abs o=%.2e ht=%.2e" % (eo, eh))


@pytest.mark.parametrize("gate", ["scalar", "channel"])
@pytest.mark.parametrize("D,T", [(64, 70), (128, 130)])
def test_prefill_recurrent_fp32(gate, D, T):
    announce("prefill fp32 %s D=%d T=%d" % (gate, D, T))
    x = synthetic.prefill_inputs(2, T, 3, D, torch.float32, gate, seed=21, device=DEV)
    o, ht = run_prefill(x, scale=0.5)
    check_prefill(x, o, ht, torch.float32, scale=0.5)


@pytest.mark.parametrize("gate", ["scalar", "channel"])
@pytest.mark.parametrize("D,T", [(64, 3), (64, 70), (128, 9), (128, 33)])
def test_prefill_recurrent_fp32_without_final_state(gate, D, T):
    """Without a final state the fp32 prefill runs the one-workgroup kernel
    (inputs loaded four tokens ahead; T < 4 and T not a multiple of 4 take
    its tail loop), with a final state the token kernel: both against the
    oracle, and their outputs against each other."""
    announce("prefill fp32 %s D=%d T=%d, no final state" % (gate, D, T))
    x = synthetic.prefill_inputs(2, T, 3, D, torch.float32, gate, seed=23, device=DEV)
    o, ht = gdr.prefill(x["q"], x["k"], x["v"], x["g"], x["beta"], h0=x["h0"], scale=0.5,
                        output_final_state=False)
    sync()
    assert ht is None
    o_ref, _ = oracle.forward(x["q"], x["k"], x["v"], x["g"], x["beta"], h0=x["h0"], scale=0.5)
    assert_close(o, o_ref, torch.float32, "o")
    o2, _ = run_prefill(x, scale=0.5)
    assert_close(o, o2, torch.float32, "o, the two kernels")


@pytest.mark.parametrize("gate", ["scalar", "channel"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("T", [1, 17, 64, 65, 200, 320])
def test_prefill_chunked_bf16(gate, D, T):
    announce("prefill bf16 %s D=%d T=%d" % (gate, D, T))
    x = synthetic.prefill_inputs(2, T, 3, D, torch.bfloat16, gate, seed=31 + T,
                                 device=DEV)
    o, ht = run_prefill(x, scale=0.9)
    eo, eh = check_prefill(x, o, ht, torch.bfloat16, scale=0.9)
    announce("  rel-fro o=%.2e ht=%.2e" % (eo, eh))


def test_prefill_chunked_bf16_zero_h0_many_heads():
    announce("prefill bf16 channel zero h0 B=1 T=256 H=9")
    x = synthetic.prefill_inputs(1, 256, 9, 128, torch.bfloat16, "channel", seed=41,
                                 h0=False, device=DEV)
    o, ht = run_prefill(x)
    check_prefill(x, o, ht, torch.bfloat16)


@pytest.mark.parametrize("dt", ["fp32", "bf16"])
def test_prefill_T0_returns_h0(dt):
    x = synthetic.prefill_inputs(2, 0, 2, 128, DTYPES[dt], "channel", seed=5, device=DEV)
    o, ht = run_prefill(x)
    assert o.numel() == 0
    assert torch.equal(ht, x["h0"])
    x["h0"] = None
    o, ht = run_prefill(x)
    assert bool((ht == 0).all())


@pytest.mark.parametrize("dt", ["fp32", "bf16"])
def test_prefill_inplace_resume(dt):
    """ht == h0 aliasing, and resume: 2 calls (split at 77) == 1 call."""
    announce("prefill in-place resume %s" % dt)
    x = synthetic.prefill_inputs(2, 160, 2, 128, DTYPES[dt], "scalar", seed=6, device=DEV)
    o_full, ht_full = run_prefill(x)
    st = x["h0"].clone()
    parts = []
    for lo, hi in ((0, 77), (77, 160)):
        sl = {n: x[n][:, lo:hi].contiguous() for n in ("q", "k", "v", "g", "beta")}
        o, _ = gdr.prefill(sl["q"], sl["k"], sl["v"], sl["g"], sl["beta"], h0=st, ht=st)
        parts.append(o)
    sync()
    o_ref, ht_ref = oracle.forward(x["q"], x["k"], x["v"], x["g"], x["beta"], h0=x["h0"])
    assert_close(torch.cat(parts, 1), o_ref, DTYPES[dt], "o split")
    assert_close(st, ht_ref, DTYPES[dt], "ht split")


@pytest.mark.parametrize("gate", ["scalar", "channel"])
@pytest.mark.parametrize("wide", [False, True])
def test_prefill_deterministic(gate, wide):
    """Run to run, bit for bit: a race on LDS or a reordered reduction would
    show here.  Scalar gate: the chunk-local kernel and the recurrence;
    channel gate: the plain pass, and (wide) the reference pass as well."""
    x = synthetic.prefill_inputs(2, 300, 4, 128, torch.bfloat16, gate, seed=8, device=DEV)
    if wide:
        x["g"][:, 100:120] = -9.0
    o1, h1 = run_prefill(x)
    for _ in range(3):
        o2, h2 = run_prefill(x)
        assert torch.equal(o1, o2) and torch.equal(h1, h2)


@pytest.mark.parametrize("gate", ["scalar", "channel"])
def test_prefill_varlen_deterministic(gate):
    """The packed form (longest-first schedule, chunk offsets on the device)
    bit for bit from run to run, at the packed workload's length mix."""
    lens = synthetic.varlen_lengths(943)
    lens = [max(1, l // 16) for l in lens]          # the same mix, 1/16 of the tokens
    x = synthetic.varlen_inputs(lens, 4, 128, torch.bfloat16, gate, seed=10, device=DEV)
    runs = []
    for _ in range(3):
        runs.append(gdr.prefill_varlen(x["q"], x["k"], x["v"], x["g"], x["beta"], x["cu_seqlens"],
                                       h0=x["h0"], cu_seqlens_host=x["cu_seqlens_host"]))
        sync()
    for o, h in runs[1:]:
        assert torch.equal(runs[0][0], o) and torch.equal(runs[0][1], h)


def test_prefill_equal_channel_gates_match_scalar_gate():
    announce("KDA with equal channel gates vs GDN (bf16)")
    x = synthetic.prefill_inputs(2, 200, 3, 128, torch.bfloat16, "scalar", seed=9, device=DEV)
    oa, ha = run_prefill(x)
    xc = dict(x)
    xc["g"] = x["g"][..., None].expand(*x["g"].shape, 128).contiguous()
    ob, hb = run_prefill(xc)
    assert_close(ob, oa.float(), torch.bfloat16, "o")
    assert_close(hb, ha, torch.bfloat16, "ht")


@pytest.mark.parametrize("gate", ["scalar", "channel"])
def test_decode_steps_match_prefill(gate):
    """T decode steps from h0 give the prefill's outputs and final state."""
    announce("decode x T vs prefill %s" % gate)
    T = 40
    x = synthetic.prefill_inputs(2, T, 3, 128, torch.bfloat16, gate, seed=10, device=DEV)
    o_p, ht_p = run_prefill(x)
    st = x["h0"].clone()
    outs = []
    for t in range(T):
        one = {n: x[n][:, t].contiguous() for n in ("q", "k", "v", "g", "beta")}
        outs.append(gdr.decode_step(one["q"], one["k"], one["v"], one["g"], one["beta"], st))
    sync()
    assert_close(torch.stack(outs, 1), o_p.float(), torch.bfloat16, "o")
    assert_close(st, ht_p, torch.bfloat16, "ht")


def test_prefill_guard_bands():
    """Writes stay inside o and ht: canaries around both are untouched."""
    x = synthetic.prefill_inputs(1, 100, 2, 128, torch.bfloat16, "channel", seed=12, device=DEV)
    pad = 4096
    n_o = x["v"].numel()
    n_h = x["h0"].numel()
    need = gdr.workspace_bytes(torch.bfloat16, True, 1, 100, 2)
    o_buf = torch.full((n_o + 2 * pad,), 3.0, device=DEV, dtype=torch.bfloat16)
    h_buf = torch.full((n_h + 2 * pad,), 5.0, device=DEV, dtype=torch.float32)
    w_buf = torch.full((need + 2 * pad,), 0xA5, device=DEV, dtype=torch.uint8)
    lib = gdr._load()
    rc = lib.gdr_prefill_chunked(
        1, 1, 1, 100, 2, 128, 128, 64, ctypes.c_float(1.0),
        x["q"].data_ptr(), x["k"].data_ptr(), x["v"].data_ptr(), x["g"].data_ptr(),
        x["beta"].data_ptr(), x["h0"].data_ptr(), o_buf.data_ptr() + 2 * pad,
        h_buf.data_ptr() + 4 * pad, w_buf.data_ptr() + pad, need,
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == 0, lib.gdr_last_error()
    sync()
    assert bool((o_buf[:pad] == 3.0).all()) and bool((o_buf[pad + n_o:] == 3.0).all())
    assert bool((h_buf[:pad] == 5.0).all()) and bool((h_buf[pad + n_h:] == 5.0).all())
    assert bool((w_buf[:pad] == 0xA5).all()) and bool((w_buf[pad + need:] == 0xA5).all())
    # without the workspace the call is refused before anything is launched
    rc = lib.gdr_prefill_chunked(
        1, 1, 1, 100, 2, 128, 128, 64, ctypes.c_float(1.0),
        x["q"].data_ptr(), x["k"].data_ptr(), x["v"].data_ptr(), x["g"].data_ptr(),
        x["beta"].data_ptr(), x["h0"].data_ptr(), o_buf.data_ptr() + 2 * pad,
        h_buf.data_ptr() + 4 * pad, None, 0,
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc != 0 and b"workspace" in lib.gdr_last_error()
    o_ref, ht_ref = oracle.forward(x["q"], x["k"], x["v"], x["g"], x["beta"], h0=x["h0"])
    assert_close(o_buf[pad:pad + n_o].view(x["v"].shape), o_ref, torch.bfloat16, "o")


@pytest.mark.parametrize("gate", ["scalar", "channel"])
def test_prefill_strong_decay(gate):
    """Gates near the documented bound: about -50 per 64 tokens, so the
    in-chunk decay factors span ~20 orders of magnitude."""
    x = synthetic.prefill_inputs(1, 200, 2, 128, torch.bfloat16, gate, seed=21,
                                 device=DEV, gate_scale=1.0)
    announce("strong decay %s: min gate sum over the first chunk %.1f"
             % (gate, float(x["g"][0, :64].sum(0).min())))
    o, ht = run_prefill(x)
    check_prefill(x, o, ht, torch.bfloat16)


@pytest.mark.parametrize("gate", ["scalar", "channel"])
def test_prefill_decay_at_the_documented_limit(gate):
    """A constant gate of -75/64 per token puts the cumulative log decay of
    every full chunk at -75, just inside the range where the channel gate's
    first pass factors a chunk from its first token (e^80): the chunk's
    e^{+-b} factors span 65 orders of magnitude and the outputs must still
    meet the bf16 bar."""
    x = synthetic.prefill_inputs(1, 200, 2, 128, torch.bfloat16, gate, seed=23, device=DEV)
    x["g"] = torch.full_like(x["g"], -75.0 / 64.0)
    announce("decay at the limit %s: gate sum per chunk %.1f"
             % (gate, float(x["g"][0, :64].sum(0).min())))
    o, ht = run_prefill(x)
    assert bool(torch.isfinite(o.float()).all()) and bool(torch.isfinite(ht).all())
    eo, eh = check_prefill(x, o, ht, torch.bfloat16)
    announce("  rel-fro o=%.2e ht=%.2e" % (eo, eh))


@pytest.mark.parametrize("gate", ["scalar", "channel"])
@pytest.mark.parametrize("spread", [0.0, 0.03, 0.3])
def test_prefill_unit_beta_collinear_keys(gate, spread):
    """The in-chunk inverse (I + diag(beta) A)^{-1} at its least favourable
    inputs: beta = 1, no decay (a = 1) and unit keys that all lie within
    `spread` of one direction, so the strictly lower part of diag(beta) A
    has entries up to 1 (exactly 1 for spread 0, where the inverse is
    bidiagonal and each token overwrites the previous one's value).  The
    kernels form the inverse from bf16 operands; the outputs must still meet
    the bf16 bar against the fp64 oracle, row by row."""
    announce("unit beta, collinear keys %s spread=%g" % (gate, spread))
    B, T, H, D = 1, 200, 2, 128
    x = synthetic.prefill_inputs(B, T, H, D, torch.bfloat16, gate, seed=27, device=DEV)
    gen = torch.Generator().manual_seed(28)
    u = torch.randn(H, D, generator=gen, dtype=torch.float64)
    k = u[None, None] + spread * torch.randn(B, T, H, D, generator=gen, dtype=torch.float64)
    k = k / k.norm(dim=-1, keepdim=True)
    x["k"] = k.to(torch.bfloat16).to(DEV)
    x["beta"] = torch.ones_like(x["beta"])
    x["g"] = torch.zeros_like(x["g"])
    o, ht = run_prefill(x)
    assert bool(torch.isfinite(o.float()).all()) and bool(torch.isfinite(ht).all())
    eo, eh = check_prefill(x, o, ht, torch.bfloat16)
    announce("  rel-fro o=%.2e ht=%.2e" % (eo, eh))


def test_prefill_guard_bands_scalar_gate_workspace():
    """Scalar gate (prep and recurrence kernels): canaries around o, ht and
    the exactly sized workspace stay untouched."""
    B, T, H = 2, 150, 3
    x = synthetic.prefill_inputs(B, T, H, 128, torch.bfloat16, "scalar", seed=22, device=DEV)
    pad = 4096
    n_o, n_h = x["v"].numel(), x["h0"].numel()
    need = gdr.workspace_bytes(torch.bfloat16, False, B, B * T, H)
    o_buf = torch.full((n_o + 2 * pad,), 3.0, device=DEV, dtype=torch.bfloat16)
    h_buf = torch.full((n_h + 2 * pad,), 5.0, device=DEV, dtype=torch.float32)
    w_buf = torch.full((need + 2 * pad,), 0xA5, device=DEV, dtype=torch.uint8)
    lib = gdr._load()
    rc = lib.gdr_prefill_chunked(
        1, 0, B, T, H, 128, 128, 64, ctypes.c_float(1.0),
        x["q"].data_ptr(), x["k"].data_ptr(), x["v"].data_ptr(), x["g"].data_ptr(),
        x["beta"].data_ptr(), x["h0"].data_ptr(), o_buf.data_ptr() + 2 * pad,
        h_buf.data_ptr() + 4 * pad, w_buf.data_ptr() + pad, need,
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == 0, lib.gdr_last_error()
    sync()
    assert bool((o_buf[:pad] == 3.0).all()) and bool((o_buf[pad + n_o:] == 3.0).all())
    assert bool((h_buf[:pad] == 5.0).all()) and bool((h_buf[pad + n_h:] == 5.0).all())
    assert bool((w_buf[:pad] == 0xA5).all()) and bool((w_buf[pad + need:] == 0xA5).all())
    o_ref, ht_ref = oracle.forward(x["q"], x["k"], x["v"], x["g"], x["beta"], h0=x["h0"])
    assert_close(o_buf[pad:pad + n_o].view(x["v"].shape), o_ref, torch.bfloat16, "o")
    assert_close(h_buf[pad:pad + n_h].view(x["h0"].shape), ht_ref, torch.bfloat16, "ht")


# ----------------------------------------------------------------- varlen
@pytest.mark.parametrize("dt", ["fp32", "bf16"])
@pytest.mark.parametrize("gate", ["scalar", "channel"])
def test_prefill_varlen(dt, gate):
    lens = [130, 0, 1, 64, 300, 17, 65]
    announce("varlen %s %s lens=%s" % (dt, gate, lens))
    x = synthetic.varlen_inputs(lens, 3, 128, DTYPES[dt], gate, seed=13, device=DEV)
    o, ht = gdr.prefill_varlen(x["q"], x["k"], x["v"], x["g"], x["beta"],
                               x["cu_seqlens"], h0=x["h0"],
                               cu_seqlens_host=x["cu_seqlens_host"])
    sync()
    o_ref, ht_ref = oracle.forward(x["q"], x["k"], x["v"], x["g"], x["beta"],
                                   h0=x["h0"], cu_seqlens=x["cu_seqlens_host"])
    assert_close(o, o_ref, DTYPES[dt], "o")
    assert_close(ht, ht_ref, DTYPES[dt], "ht")
    # the empty sequence keeps its initial state exactly
    assert torch.equal(ht[1], x["h0"][1])


@pytest.mark.parametrize("gate", ["scalar", "channel"])
def test_prefill_varlen_many_short_sequences(gate):
    """300 packed sequences (the chunk offsets take several sequences per
    scan thread), lengths 0..130 including empty ones, no h0."""
    rng = np.random.default_rng(23)
    lens = [int(v) for v in rng.integers(0, 131, size=300)]
    lens[5] = lens[77] = 0
    announce("varlen %s: %d sequences, %d tokens" % (gate, len(lens), sum(lens)))
    x = synthetic.varlen_inputs(lens, 2, 128, torch.bfloat16, gate, seed=23, h0=False,
                                device=DEV)
    o, ht = gdr.prefill_varlen(x["q"], x["k"], x["v"], x["g"], x["beta"],
                               x["cu_seqlens"], cu_seqlens_host=x["cu_seqlens_host"])
    sync()
    o_ref, ht_ref = oracle.forward(x["q"], x["k"], x["v"], x["g"], x["beta"],
                                   cu_seqlens=x["cu_seqlens_host"])
    assert_close(o, o_ref, torch.bfloat16, "o")
    assert_close(ht, ht_ref, torch.bfloat16, "ht")
    assert not bool(ht[5].any()) and not bool(ht[77].any())


@pytest.mark.parametrize("gate", ["scalar", "channel"])
def test_prefill_varlen_equals_fixed_when_uniform(gate):
    x = synthetic.prefill_inputs(3, 150, 2, 128, torch.bfloat16, gate, seed=14, device=DEV)
    o1, h1 = run_prefill(x)
    cu = torch.arange(4, device=DEV, dtype=torch.int32) * 150
    flat = {n: x[n].reshape(450, *x[n].shape[2:]) for n in ("q", "k", "v", "g", "beta")}
    o2, h2 = gdr.prefill_varlen(flat["q"], flat["k"], flat["v"], flat["g"], flat["beta"],
                                cu, h0=x["h0"])
    sync()
    assert torch.equal(o1.reshape(450, 2, 128), o2) and torch.equal(h1, h2)
