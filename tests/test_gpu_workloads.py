"""GPU parity at the five workloads' full sizes, in the launch configuration
bench.py times.  The kernels run on the whole workload and the fp64 oracle
recomputes all of it: every (sequence, head) of the prefill workloads (the
packed one streamed eight heads at a time to bound host memory), whole GDN
and KDA layers of the placement decode plus slots sampled over all its
recurrent layers.  Each tensor meets the bar as a whole, row by row, and
(prefill) per (sequence, head); FA/SWA slots stay untouched."""
import numpy as np
import pytest
import torch

import gated_delta_rule_44_amd as gdr
import oracle
from gated_delta_rule_44_amd import synthetic
from tests.conftest import gpu_available
from tests.gpu_util import announce, assert_close, assert_pairs_close, heads_first

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]
DEV = torch.device("cuda:0")


def sync():
    torch.cuda.synchronize(DEV)


def test_gdn_recurrent_fp32_B1_H1_T64_d64():
    w = synthetic.WORKLOADS[0]
    announce("workload %s" % w.name)
    x = synthetic.prefill_inputs(w.B, w.T, w.H, w.D, w.dtype, w.gate, seed=w.seed,
                                 h0=w.h0, device=DEV)
    o, ht = gdr.prefill(x["q"], x["k"], x["v"], x["g"], x["beta"], h0=x["h0"])
    sync()
    o_ref, ht_ref = oracle.forward(x["q"], x["k"], x["v"], x["g"], x["beta"], h0=None)
    eo = assert_close(o, o_ref, torch.float32, "o")
    eh = assert_close(ht, ht_ref, torch.float32, "ht")
    announce("  max-abs o=%.2e ht=%.2e" % (eo, eh))


def _full_prefill(w):
    x = synthetic.prefill_inputs(w.B, w.T, w.H, w.D, w.dtype, w.gate, seed=w.seed,
                                 h0=w.h0, device=DEV)
    o, ht = gdr.prefill(x["q"], x["k"], x["v"], x["g"], x["beta"], h0=x["h0"])
    sync()
    announce("  kernels done; fp64 oracle over all %d (sequence, head) pairs" % (w.B * w.H))
    o_ref, ht_ref = oracle.forward(x["q"], x["k"], x["v"], x["g"], x["beta"], h0=x["h0"])
    eo = assert_close(o, o_ref, torch.bfloat16, "o")
    eh = assert_close(ht, ht_ref, torch.bfloat16, "ht")
    po = assert_pairs_close(heads_first(o), heads_first(o_ref), "o")
    ph = assert_pairs_close(ht.reshape(w.B * w.H, w.D, w.D), ht_ref.reshape(w.B * w.H, w.D, w.D), "ht")
    announce("  rel-fro o=%.2e ht=%.2e; worst pair o=%.2e ht=%.2e" % (eo, eh, po, ph))


def test_gdn_prefill_B4_H16_T4096():
    w = synthetic.WORKLOADS[1]
    announce("workload %s" % w.name)
    _full_prefill(w)


def test_kda_prefill_B2_H32_T8192():
    w = synthetic.WORKLOADS[2]
    announce("workload %s" % w.name)
    _full_prefill(w)


def test_placement_decode_L48_B256_H32():
    w = synthetic.WORKLOADS[3]
    announce("workload %s" % w.name)
    place = synthetic.placement(0, w.L)
    x = synthetic.decode_inputs(w.L, w.B, w.H, w.D, w.dtype, place=place, seed=w.seed,
                                device=DEV)
    rec = [l for l in range(w.L) if place[l] in (synthetic.GDN, synthetic.KDA)]
    other = [l for l in range(w.L) if l not in rec]
    rng = np.random.default_rng(3)
    samples = [(int(rng.choice(rec)), int(rng.integers(w.B)), int(rng.integers(w.H)))
               for _ in range(48)]
    before = {s: x["pool"][s].clone() for s in samples}
    # one whole GDN layer and one whole KDA layer are checked slot by slot
    whole = [next(i for i in rec if place[i] == c) for c in (synthetic.GDN, synthetic.KDA)]
    before_layer = {l: x["pool"][l].clone() for l in whole}
    untouched = x["pool"][other]          # advanced indexing copies
    o = torch.full_like(x["v"], -5.0)
    gdr.decode_placement(place, x["q"], x["k"], x["v"], x["g"], x["beta"], x["pool"], o=o)
    sync()
    assert torch.equal(x["pool"][other], untouched), "FA/SWA state slots changed"
    assert bool((o[other] == -5.0).all()), "FA/SWA output slots written"
    del untouched
    got_o, ref_o, got_s, ref_s = [], [], [], []
    for (l, b, h) in samples:
        g = x["g"][l, b:b + 1, h:h + 1]
        if place[l] == synthetic.GDN:
            g = g[..., 0]
        oo, ss = oracle.decode(x["q"][l, b:b + 1, h:h + 1], x["k"][l, b:b + 1, h:h + 1],
                               x["v"][l, b:b + 1, h:h + 1], g,
                               x["beta"][l, b:b + 1, h:h + 1], before[(l, b, h)][None, None])
        got_o.append(o[l, b, h].float().cpu().numpy())
        ref_o.append(oo[0, 0])
        got_s.append(x["pool"][l, b, h].cpu().numpy())
        ref_s.append(ss[0, 0])
    eo = assert_close(np.stack(got_o), np.stack(ref_o), torch.bfloat16, "o samples")
    es = assert_close(np.stack(got_s), np.stack(ref_s), torch.bfloat16, "state samples")
    announce("  48 sampled slots: rel-fro o=%.2e state=%.2e, max-abs state=%.2e"
             % (eo, es, float(np.abs(np.stack(got_s) - np.stack(ref_s)).max())))
    # the whole GDN layer and the whole KDA layer, every (b, h) slot
    for l in whole:
        code = place[l]
        g = x["g"][l] if code == synthetic.KDA else x["g"][l][..., 0]
        oo, ss = oracle.decode(x["q"][l], x["k"][l], x["v"][l], g, x["beta"][l], before_layer[l])
        eo = assert_close(o[l], oo, torch.bfloat16, "o layer %d" % l)
        es = assert_close(x["pool"][l], ss, torch.bfloat16, "state layer %d" % l)
        assert float(np.abs(x["pool"][l].cpu().numpy() - ss).max()) < 1e-5
        announce("  whole %s layer %d (%d slots): rel-fro o=%.2e state=%.2e"
                 % ("GDN" if code == synthetic.GDN else "KDA", l, w.B * w.H, eo, es))


def test_kda_varlen_N16_H32():
    w = synthetic.WORKLOADS[4]
    announce("workload %s" % w.name)
    lens = synthetic.varlen_lengths(943)
    x = synthetic.varlen_inputs(lens, w.H, w.D, w.dtype, w.gate, seed=w.seed, device=DEV)
    o, ht = gdr.prefill_varlen(x["q"], x["k"], x["v"], x["g"], x["beta"], x["cu_seqlens"],
                               h0=x["h0"], cu_seqlens_host=x["cu_seqlens_host"])
    sync()
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(ht).all())
    cu = x["cu_seqlens_host"]
    N = len(lens)
    worst = [0.0, 0.0]
    for h0 in range(0, w.H, 8):            # eight heads at a time
        hs = slice(h0, h0 + 8)
        sl = {k: x[k][:, hs].contiguous() for k in ("q", "k", "v", "g", "beta")}
        o_ref, ht_ref = oracle.forward(sl["q"], sl["k"], sl["v"], sl["g"], sl["beta"],
                                       h0=x["h0"][:, hs].contiguous(), cu_seqlens=cu)
        eo = assert_close(o[:, hs], o_ref, torch.bfloat16, "o heads %d.." % h0)
        eh = assert_close(ht[:, hs], ht_ref, torch.bfloat16, "ht heads %d.." % h0)
        og = o[:, hs].float().cpu().numpy()
        for n in range(N):                 # each (sequence, head) on its own
            lo, hi = int(cu[n]), int(cu[n + 1])
            worst[0] = max(worst[0], assert_pairs_close(np.moveaxis(og[lo:hi], 1, 0),
                                                        np.moveaxis(o_ref[lo:hi], 1, 0),
                                                        "o n=%d heads %d.." % (n, h0)))
        worst[1] = max(worst[1], assert_pairs_close(ht[:, hs].reshape(N * 8, w.D, w.D),
                                                    ht_ref.reshape(N * 8, w.D, w.D), "ht"))
        announce("  heads %d..%d: rel-fro o=%.2e ht=%.2e" % (h0, h0 + 7, eo, eh))
    announce("  worst (sequence, head): o=%.2e ht=%.2e" % tuple(worst))
