"""GPU parity at the five workloads' full sizes, in the launch configuration
bench.py times.  The kernels run on the whole workload; the fp64 oracle
recomputes sampled (sequence, head) pairs or (layer, b, h) slots one by
one, and whole-tensor properties (finite values, untouched slots) are
checked everywhere."""
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


def _sampled_prefill(w, pairs):
    x = synthetic.prefill_inputs(w.B, w.T, w.H, w.D, w.dtype, w.gate, seed=w.seed,
                                 h0=w.h0, device=DEV)
    o, ht = gdr.prefill(x["q"], x["k"], x["v"], x["g"], x["beta"], h0=x["h0"])
    sync()
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(ht).all())
    for b, h in pairs:
        sl = {n: x[n][b:b + 1, :, h:h + 1].contiguous() for n in ("q", "k", "v", "g", "beta")}
        h0 = None if x["h0"] is None else x["h0"][b:b + 1, h:h + 1].contiguous()
        o_ref, ht_ref = oracle.forward(sl["q"], sl["k"], sl["v"], sl["g"], sl["beta"], h0=h0)
        eo = assert_close(o[b:b + 1, :, h:h + 1], o_ref, torch.bfloat16, "o[%d,:,%d]" % (b, h))
        eh = assert_close(ht[b:b + 1, h:h + 1], ht_ref, torch.bfloat16, "ht[%d,%d]" % (b, h))
        announce("  (b=%d,h=%d) rel-fro o=%.2e ht=%.2e" % (b, h, eo, eh))


def test_gdn_prefill_B4_H16_T4096():
    w = synthetic.WORKLOADS[1]
    announce("workload %s" % w.name)
    _sampled_prefill(w, [(0, 0), (1, 7), (3, 15)])


def test_kda_prefill_B2_H32_T8192():
    w = synthetic.WORKLOADS[2]
    announce("workload %s" % w.name)
    _sampled_prefill(w, [(0, 0), (1, 31)])


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
    # shortest sequences (several heads) and one head of the longest one
    order = np.argsort(lens)
    picks = [(int(order[0]), 0), (int(order[0]), 31), (int(order[1]), 5),
             (int(order[-1]), 17)]
    for n, h in picks:
        lo, hi = int(cu[n]), int(cu[n + 1])
        sl = {k: x[k][lo:hi, h:h + 1].contiguous() for k in ("q", "k", "v", "g", "beta")}
        o_ref, ht_ref = oracle.forward(sl["q"], sl["k"], sl["v"], sl["g"], sl["beta"],
                                       h0=x["h0"][n:n + 1, h:h + 1].contiguous(),
                                       cu_seqlens=np.array([0, hi - lo]))
        eo = assert_close(o[lo:hi, h:h + 1], o_ref, torch.bfloat16, "o n=%d h=%d" % (n, h))
        eh = assert_close(ht[n:n + 1, h:h + 1], ht_ref, torch.bfloat16, "ht n=%d h=%d" % (n, h))
        announce("  (n=%d len=%d h=%d) rel-fro o=%.2e ht=%.2e" % (n, hi - lo, h, eo, eh))
