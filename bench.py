#!/usr/bin/env python3
"""Throughput of the gated delta-rule hot path on one MI355X.

Headline (the single JSON line's `value`): chunked prefill tokens/s on the
Gated DeltaNet workload B=4, H=16, T=4096, d_k=d_v=128, bf16 q/k/v, fp32
gates/beta/initial state, chunk 64 (one gdr_prefill_chunked launch per
step, outputs plus final states).  Inputs are resident in HBM before timing
and rotate over three input sets so that a step cannot be served from the
256 MB last-level cache.

The same line carries:
  roofline      the prefill call's algorithmic HBM bytes over its average
                time (HIP events on the launch stream), against 8 TB/s.  One
                gdr_prefill_chunked call is two back-to-back kernels on that
                stream: prep_kernel (the chunk-local inverses) and
                chain_kernel (the recurrence, the dominant one); `traffic`
                is the measured bytes per call from rocprofv3
                FETCH_SIZE/WRITE_SIZE counters summed over both, when given
  cpu_baseline  the fp64 oracle on the host cores, on a bounded sample of
                the same workload (the first tokens of every sequence/head)
  secondary     the other hot-path entry points measured in the same run:
                KDA prefill, the placement-driven decode step (state-update
                GB/s and % of HBM peak), the packed variable-length KDA
                prefill, the drafted decode (4 tokens with per-token
                checkpoints, then the commit of the accepted prefixes) on a
                slot-indexed pool, the packed KDA prefill through a pool, and
                the GDN and KDA prefill on raw projections (fused q/k
                normalisation, beta and gate from bf16 logits), and the
                backward of the GDN and KDA prefill workloads and of the
                packed KDA workload, and the GDN backward with every
                (sequence, head) past the chunk form's range (g = -4 per
                token: the exact token-level path).

Times: each step is bracketed by HIP events on the launch stream; `value`
and `ms_per_step` come from the median step, `roofline.achieved` from the
mean (the average call time, as rocprofv3 reports kernel averages).
Defaults: 100 warmup steps and 200 timed steps (a fifth of each for the
decode and varlen workloads).  The GPU clock ramps up over the first ~25 ms
of sustained load (headline calls 0-100 take 126-133 us, calls past 200
117 us), so before each workload's W warm-up calls come untimed calls
filling `--settle-ms` (default 40) ms of GPU time; the line reports the
headline's as `clock_settle_calls`.
The secondary list also carries the latency of one fp32 call on the GDN
recurrent workload (B=1 H=1 T=64 d=64), and the oracle's rate on the other
workloads in full beside the GPU's.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--settle-ms MS]
                       [--only-headline] [--no-cpu-baseline]
                       [--only {kda_prefill,decode,varlen,draft,varlen_pool,fused_gdn,fused_kda,
                                backward_gdn,backward_kda,backward_kda_varlen}]
                       (one workload, for profiling)
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "GDN/KDA prefill tokens/s + decode state-update GB/s (% of HBM peak), 1 GPU"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_TFLOPS = 2500.0
D, C = 128, 64
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_DIR = os.path.join(ROOT, "gated_delta_rule_44_amd", "csrc")


def sources_sha256(names):
    """sha256 over the named kernel source files, in the order given."""
    import hashlib
    h = hashlib.sha256()
    for n in names:
        h.update(open(os.path.join(KERNEL_DIR, n), "rb").read())
    return h.hexdigest()


def measured_traffic(workload):
    """HBM bytes per call of a workload (all its kernels) from rocprofv3
    FETCH_SIZE / WRITE_SIZE counters, scaled by the factors a plain copy of
    known size gives (profiles/traffic.json), and their ratio to the
    algorithmic bytes; None when the counters were taken on another version
    of the sources the workload's kernels are built from (each entry names
    them and their hash)."""
    try:
        rec = json.load(open(TRAFFIC_FILE))
        w = rec.get("workloads", {}).get(workload)
        if not w or "bytes_per_call" not in w or "sources" not in w:
            return None
        if sources_sha256(w["sources"]) != w.get("sources_sha256"):
            return None
    except (OSError, ValueError):
        return None
    return {"bytes_per_call": w["bytes_per_call"],
            "over_algorithmic": w["traffic_over_algorithmic"]}


def prefill_bytes(tokens_heads, units, gate):
    """Algorithmic HBM bytes: q,k,v,o in bf16, beta and the gate in fp32 per
    token-head; initial and final fp32 state per (sequence, head)."""
    per_tok = 3 * D * 2 + D * 2 + 4 + (4 * D if gate == "channel" else 4)
    return tokens_heads * per_tok + units * 2 * D * D * 4


def prefill_flops(tokens_heads):
    """Algorithmic flops of the chunked form per token-head (causal
    triangles only): 5Cd + 6d^2 + C^2/3."""
    return tokens_heads * (5 * C * D + 6 * D * D + C * C / 3.0)


def decode_bytes(head_steps, gate_bytes):
    """Per head-step: fp32 state read + write, q,k,v in bf16, o bf16, beta,
    gate."""
    return head_steps * (2 * D * D * 4 + 3 * D * 2 + D * 2 + 4) + gate_bytes


LAST_MEAN_MS = [0.0]
SETTLE_MS = [40.0]          # untimed GPU time before each workload's warm-up
LAST_SETTLE_CALLS = [0]


def timed(fn, steps, warmup, stream):
    """Median ms per step over `steps` timed steps, each bracketed by HIP
    events on the launch stream (the mean is kept in LAST_MEAN_MS[0]).
    Before the `warmup` calls, untimed calls fill about SETTLE_MS[0] ms of
    GPU time (their count is kept in LAST_SETTLE_CALLS[0]): the GPU clock
    ramps up over the first ~25 ms of sustained load."""
    import time
    import torch
    n, batch = 0, 1
    if SETTLE_MS[0] > 0:
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        while n < 20000:
            for _ in range(batch):
                fn(n)
                n += 1
            torch.cuda.synchronize()
            if time.perf_counter() - t0 >= SETTLE_MS[0] * 1e-3:
                break
            batch = min(2 * batch, 64)
    LAST_SETTLE_CALLS[0] = n
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    ev[0].record(stream)
    for i in range(steps):
        fn(i)
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    per = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(steps))
    LAST_MEAN_MS[0] = ev[0].elapsed_time(ev[steps]) / steps
    mid = steps // 2
    return per[mid] if steps % 2 else 0.5 * (per[mid - 1] + per[mid])


def bench_prefill(gdr, synthetic, torch, dev, B, T, H, gate, seed, steps, warmup,
                  h0=True, sets=3):
    xs = [synthetic.prefill_inputs(B, T, H, D, torch.bfloat16, gate, seed=seed + i,
                                   h0=h0, device=dev) for i in range(sets)]
    outs = [(torch.empty_like(x["v"]), torch.empty((B, H, D, D), device=dev,
                                                     dtype=torch.float32)) for x in xs]
    lib = gdr._load()
    import ctypes
    stream = torch.cuda.current_stream(dev)
    sp = ctypes.c_void_p(stream.cuda_stream)
    gk = 1 if gate == "channel" else 0
    nbytes = gdr.workspace_bytes(torch.bfloat16, gate == "channel", B, B * T, H)
    ws = torch.empty(max(nbytes, 1), device=dev, dtype=torch.uint8)
    args = []
    for x, (o, ht) in zip(xs, outs):
        args.append([1, gk, B, T, H, D, D, C, ctypes.c_float(1.0)] +
                    [ctypes.c_void_p(t.data_ptr()) if t is not None else None
                     for t in (x["q"], x["k"], x["v"], x["g"], x["beta"], x["h0"], o, ht, ws)]
                    + [ctypes.c_size_t(nbytes), sp])

    def step(i):
        rc = lib.gdr_prefill_chunked(*args[i % sets])
        if rc:
            raise RuntimeError(lib.gdr_last_error().decode())
    ms = timed(step, steps, warmup, stream)
    del xs, outs, ws
    return ms


def bench_recurrent(gdr, synthetic, torch, dev, steps, warmup):
    """One fp32 call on the GDN recurrent workload (B=1, H=1, T=64, d=64,
    zero initial state): its latency."""
    x = synthetic.prefill_inputs(1, 64, 1, 64, torch.float32, "scalar", seed=1000, h0=False,
                                 device=dev)
    o = torch.empty_like(x["v"])
    ht = torch.empty((1, 1, 64, 64), device=dev, dtype=torch.float32)
    lib = gdr._load()
    import ctypes
    stream = torch.cuda.current_stream(dev)
    P = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())  # noqa: E731
    args = [0, 0, 1, 64, 1, 64, 64, C, ctypes.c_float(1.0)] + \
        [P(t) for t in (x["q"], x["k"], x["v"], x["g"], x["beta"], None, o, ht)] + \
        [None, ctypes.c_size_t(0), ctypes.c_void_p(stream.cuda_stream)]

    def step(i):
        rc = lib.gdr_prefill_chunked(*args)
        if rc:
            raise RuntimeError(lib.gdr_last_error().decode())
    return timed(step, steps, warmup, stream)


def bench_fused(gdr, synthetic, torch, dev, B, T, H, gate, seed, steps, warmup, h0=True,
                sets=3):
    """Chunked prefill on raw projections (fused preprocessing): q, k, v and
    the logits in bf16, rotating over `sets` input sets."""
    xs = [synthetic.raw_prefill_inputs(B, T, H, D, torch.bfloat16, gate, seed=seed + i,
                                       h0=h0, device=dev) for i in range(sets)]
    ht = torch.empty((B, H, D, D), device=dev, dtype=torch.float32)
    ws = torch.empty(max(gdr.fused_workspace_bytes(torch.bfloat16, gate == "channel", B, B * T, H), 1),
                     device=dev, dtype=torch.uint8)
    stream = torch.cuda.current_stream(dev)

    def step(i):
        x = xs[i % sets]
        gdr.prefill_fused(x["q"], x["k"], x["v"], x["gate_logit"], x["beta_logit"],
                          x["gate_scale"], h0=x["h0"], ht=ht, workspace=ws)
    ms = timed(step, steps, warmup, stream)
    del xs, ht, ws
    return ms


def bench_backward(gdr, synthetic, torch, dev, B, T, H, gate, seed, steps, warmup, h0=True,
                   gate_fill=None):
    """Gradients of the chunked prefill (gdr_backward_chunked): all inputs and
    the upstream gradients resident, outputs and workspace preallocated.
    gate_fill: every gate log set to this value (e.g. -4: every chunk decays
    by e^-256, so every pair takes the token-level path)."""
    x = synthetic.prefill_inputs(B, T, H, D, torch.bfloat16, gate, seed=seed, h0=h0, device=dev)
    if gate_fill is not None:
        x["g"].fill_(gate_fill)
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed + 50)
    do = torch.randn((B, T, H, D), generator=gen, device=dev).to(torch.bfloat16)
    dht = torch.randn((B, H, D, D), generator=gen, device=dev) * 0.1
    lib = gdr._load()
    import ctypes
    f32 = dict(device=dev, dtype=torch.float32)
    outs = [torch.empty((B, T, H, D), **f32) for _ in range(3)] + \
        [torch.empty(x["g"].shape, **f32), torch.empty((B, T, H), **f32),
         torch.empty((B, H, D, D), **f32)]
    nbytes = int(lib.gdr_backward_workspace_bytes(1 if gate == "channel" else 0, B, T, H, D, D))
    ws = torch.empty(nbytes, device=dev, dtype=torch.uint8)
    stream = torch.cuda.current_stream(dev)
    P = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())  # noqa: E731
    args = [1, 1 if gate == "channel" else 0, B, T, H, D, D, C, ctypes.c_float(1.0),
            P(x["q"]), P(x["k"]), P(x["v"]), P(x["g"]), P(x["beta"]), P(x["h0"]), P(do), P(dht)] + \
        [P(t) for t in outs] + [P(ws), ctypes.c_size_t(nbytes), ctypes.c_void_p(stream.cuda_stream)]

    def step(i):
        rc = lib.gdr_backward_chunked(*args)
        if rc:
            raise RuntimeError(lib.gdr_last_error().decode())
    ms = timed(step, steps, warmup, stream)
    del x, outs, ws
    return ms


def bench_backward_varlen(gdr, synthetic, torch, dev, steps, warmup):
    """Gradients of the packed KDA prefill (gdr_backward_chunked_varlen) on the
    varlen workload: 16 sequences of 512..65536 tokens, H = 32."""
    lens = synthetic.varlen_lengths(943)
    H = 32
    x = synthetic.varlen_inputs(lens, H, D, torch.bfloat16, "channel", seed=1004, device=dev)
    Tt, N = sum(lens), len(lens)
    gen = torch.Generator(device=dev)
    gen.manual_seed(1054)
    do = torch.randn((Tt, H, D), generator=gen, device=dev).to(torch.bfloat16)
    dht = torch.randn((N, H, D, D), generator=gen, device=dev) * 0.1
    lib = gdr._load()
    import ctypes
    f32 = dict(device=dev, dtype=torch.float32)
    outs = [torch.empty((Tt, H, D), **f32) for _ in range(3)] + \
        [torch.empty(x["g"].shape, **f32), torch.empty((Tt, H), **f32),
         torch.empty((N, H, D, D), **f32)]
    nbytes = int(lib.gdr_backward_varlen_workspace_bytes(1, N, Tt, H, D, D))
    ws = torch.empty(nbytes, device=dev, dtype=torch.uint8)
    stream = torch.cuda.current_stream(dev)
    P = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())  # noqa: E731
    args = [1, 1, N, Tt, H, D, D, C, ctypes.c_float(1.0), P(x["cu_seqlens"]), None,
            P(x["q"]), P(x["k"]), P(x["v"]), P(x["g"]), P(x["beta"]), P(x["h0"]), P(do), P(dht)] + \
        [P(t) for t in outs] + [P(ws), ctypes.c_size_t(nbytes), ctypes.c_void_p(stream.cuda_stream)]

    def step(i):
        rc = lib.gdr_backward_chunked_varlen(*args)
        if rc:
            raise RuntimeError(lib.gdr_last_error().decode())
    ms = timed(step, steps, warmup, stream)
    del x, outs, ws
    return ms, Tt, N


def backward_bytes(tokens_heads, units, gate, h0=True):
    """Algorithmic HBM bytes of one backward call: q, k, v, do in bf16, g and
    beta read; dq, dk, dv in fp32, dg and dbeta written, per token-head;
    h0, dht read and dh0 written per (sequence, head)."""
    gb = 4 * D if gate == "channel" else 4
    per_tok = 4 * D * 2 + gb + 4 + 3 * D * 4 + gb + 4
    return tokens_heads * per_tok + units * (3 if h0 else 2) * D * D * 4


def bench_varlen(gdr, synthetic, torch, dev, steps, warmup):
    lens = synthetic.varlen_lengths(943)
    x = synthetic.varlen_inputs(lens, 32, D, torch.bfloat16, "channel", seed=1004,
                                device=dev)
    o = torch.empty_like(x["v"])
    ht = torch.empty_like(x["h0"])
    ws = torch.empty(gdr.workspace_bytes(torch.bfloat16, True, len(lens), sum(lens), 32),
                     device=dev, dtype=torch.uint8)
    stream = torch.cuda.current_stream(dev)

    def step(i):
        gdr.prefill_varlen(x["q"], x["k"], x["v"], x["g"], x["beta"], x["cu_seqlens"],
                           h0=x["h0"], workspace=ws, ht=ht)
    ms = timed(step, steps, warmup, stream)
    tokens = sum(lens)
    del x, o, ht
    return ms, tokens, lens


def bench_decode(gdr, synthetic, torch, dev, steps, warmup):
    place = synthetic.placement(0, 48)
    x = synthetic.decode_inputs(48, 256, 32, D, torch.bfloat16, place=place,
                                seed=1003, device=dev)
    o = torch.empty_like(x["v"])
    stream = torch.cuda.current_stream(dev)

    def step(i):
        gdr.decode_placement(place, x["q"], x["k"], x["v"], x["g"], x["beta"],
                             x["pool"], o=o)
    ms = timed(step, steps, warmup, stream)
    n_gdn = int((place == synthetic.GDN).sum())
    n_kda = int((place == synthetic.KDA).sum())
    del x, o
    return ms, n_gdn, n_kda, synthetic.placement_string(place)


def bench_draft(gdr, synthetic, torch, dev, steps, warmup):
    """Drafted decode: 4 tokens for 256 sequences x 32 heads (GDN, bf16) whose
    states sit in a 512-slot pool, with a checkpoint after every token, then
    the commit of the accepted prefixes.  The two calls are timed apart."""
    B, n, H, P = 256, 4, 32, 512
    x = synthetic.prefill_inputs(B, n, H, D, torch.bfloat16, "scalar", seed=1005,
                                 h0=False, device=dev)
    pool = synthetic.pool_states(P, H, D, seed=1006, device=dev)
    slot = torch.from_numpy(synthetic.serving_slots(B, P, seed=1007)).to(dev)
    acc_np = synthetic.accepted_counts(B, n, seed=1008)
    acc = torch.from_numpy(acc_np).to(dev)
    ck = torch.empty((B, n, H, D, D), device=dev, dtype=torch.float32)
    o = torch.empty_like(x["v"])
    stream = torch.cuda.current_stream(dev)
    args = [x[k] for k in ("q", "k", "v", "g", "beta")]

    def draft(i):
        gdr.decode_tokens(*args, pool, slot=slot, checkpoints=ck, o=o)

    def commit(i):
        gdr.decode_commit(ck, acc, pool, slot=slot)
    ms_d = timed(draft, steps, warmup, stream)
    ms_c = timed(commit, steps, warmup, stream)
    kept = int((acc_np >= 1).sum())
    del x, pool, ck, o
    return ms_d, ms_c, B, n, H, kept


def bench_varlen_pool(gdr, synthetic, torch, dev, steps, warmup):
    """The KDA packed workload with its states in a 40-slot pool (each
    sequence starts from one slot and ends in another)."""
    lens = synthetic.varlen_lengths(943)
    N, H, P = len(lens), 32, 40
    x = synthetic.varlen_inputs(lens, H, D, torch.bfloat16, "channel", seed=1004,
                                h0=False, device=dev)
    pool = synthetic.pool_states(P, H, D, seed=1009, device=dev)
    import numpy as np
    h0s = np.arange(N, dtype=np.int32)
    hts = np.arange(N, 2 * N, dtype=np.int32)
    h0t, htt = torch.from_numpy(h0s).to(dev), torch.from_numpy(hts).to(dev)
    ws = torch.empty(gdr.workspace_bytes(torch.bfloat16, True, N, sum(lens), H),
                     device=dev, dtype=torch.uint8)
    stream = torch.cuda.current_stream(dev)
    args = [x[k] for k in ("q", "k", "v", "g", "beta")]

    def step(i):
        gdr.prefill_varlen_pool(*args, x["cu_seqlens"], pool, h0t, htt, workspace=ws)
    ms = timed(step, steps, warmup, stream)
    del x, pool, ws
    return ms, sum(lens)


def host_threads():
    """(threads the oracle runs on, CPUs in this process's affinity mask):
    the affinity mask, capped by OMP_NUM_THREADS when that is set."""
    aff = len(os.sched_getaffinity(0))
    try:
        omp = int(os.environ.get("OMP_NUM_THREADS", "0"))
    except ValueError:
        omp = 0
    return (min(aff, omp) if omp > 0 else aff), aff


def cpu_baseline(synthetic, torch, target_s=3.0):
    """The fp64 oracle as it stands on the host cores, on the workloads'
    inputs drawn on the host: the GDN prefill in full (the headline's;
    repeated until about target_s seconds have passed), the KDA prefill in
    full, one step of the placement decode over all its recurrent layers,
    and the packed KDA prefill at 8 of its 32 heads (its rate scaled to all
    of them).  Returns (the headline's baseline, entries for the other
    workloads)."""
    import numpy as np
    import oracle
    threads, aff = host_threads()

    def prefill_s(B, T, H, gate, seed, h0):
        x = synthetic.prefill_inputs(B, T, H, D, torch.bfloat16, gate, seed=seed, h0=h0,
                                     device="cpu")
        t0 = time.perf_counter()
        oracle.forward(x["q"], x["k"], x["v"], x["g"], x["beta"], h0=x["h0"], threads=threads)
        return time.perf_counter() - t0

    total_t, reps = 0.0, 0
    while total_t < target_s or reps == 0:
        total_t += prefill_s(4, 4096, 16, "scalar", 1001, True)
        reps += 1
    head = {"value": reps * 4 * 4096 / total_t, "unit": "tokens/s", "cores": threads,
            "host_cores": aff, "kind": "oracle",
            "sample": "GDN prefill B=4 H=16 T=4096 d=128 in full (all 64 sequence-heads), "
                      "fp64 token by token, %d pass(es), %.1f s" % (reps, total_t)}
    out = []
    t2 = prefill_s(2, 8192, 32, "channel", 1002, False)
    out.append({"workload": "kda_prefill_B2_H32_T8192_d128_bf16", "value": 2 * 8192 / t2,
                "unit": "tokens/s", "seconds": t2, "sample": "in full"})
    # placement decode: every recurrent layer of one step
    place = synthetic.placement(0, 48)
    rec = [l for l in range(48) if place[l] in (synthetic.GDN, synthetic.KDA)]
    gen = torch.Generator().manual_seed(1003)
    t3 = 0.0
    for l in rec:
        q = torch.randn((256, 32, D), generator=gen)
        q = (q / q.norm(dim=-1, keepdim=True)).to(torch.bfloat16)
        k = torch.randn((256, 32, D), generator=gen)
        k = (k / k.norm(dim=-1, keepdim=True)).to(torch.bfloat16)
        v = torch.randn((256, 32, D), generator=gen).to(torch.bfloat16)
        beta = torch.sigmoid(torch.randn((256, 32), generator=gen))
        c = 0.1 if place[l] == synthetic.GDN else 0.05
        g = -torch.nn.functional.softplus(torch.randn((256, 32, D), generator=gen)) * c
        if place[l] == synthetic.GDN:
            g = g[..., 0].contiguous()
        st = torch.randn((256, 32, D, D), generator=gen) * 0.02
        t0 = time.perf_counter()
        oracle.decode(q, k, v, g, beta, st, threads=threads)
        t3 += time.perf_counter() - t0
    out.append({"workload": "placement_decode_L48_B256_H32_d128_bf16",
                "value": 256 / t3, "unit": "tokens/s", "head_steps_per_s": len(rec) * 256 * 32 / t3,
                "seconds": t3, "sample": "one step over the %d recurrent layers (inputs of the "
                                         "same law, host-drawn)" % len(rec)})
    # packed KDA: all 16 sequences in full, 8 of the 32 heads (the work per
    # head is the same), scaled to the whole workload's tokens/s
    lens = synthetic.varlen_lengths(943)
    x = synthetic.varlen_inputs(lens, 8, D, torch.bfloat16, "channel", seed=1004, device="cpu")
    t0 = time.perf_counter()
    oracle.forward(x["q"], x["k"], x["v"], x["g"], x["beta"], h0=x["h0"],
                   cu_seqlens=x["cu_seqlens_host"], threads=threads)
    t4 = time.perf_counter() - t0
    out.append({"workload": "kda_varlen_N16_H32_d128_bf16", "value": int(np.sum(lens)) * 8 / 32 / t4,
                "unit": "tokens/s", "seconds": t4,
                "sample": "all 16 sequences (%d tokens) at 8 of the 32 heads, rate scaled to "
                          "32 heads" % int(np.sum(lens))})
    for e in out:
        e.update({"cores": threads, "host_cores": aff, "kind": "oracle"})
    return head, out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--settle-ms", type=float, default=40.0,
                    help="untimed GPU time (ms) before each workload's warm-up calls, so "
                         "that the GPU is at its steady clock when timing starts")
    ap.add_argument("--only-headline", action="store_true")
    ap.add_argument("--only", choices=["gdn_prefill", "kda_prefill", "decode", "varlen", "draft",
                                       "varlen_pool", "fused_gdn", "fused_kda", "backward_gdn",
                                       "backward_kda", "backward_kda_varlen", "recurrent",
                                       "hbm_copy"],
                    default=None,
                    help="time one secondary workload alone (for profiling)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    SETTLE_MS[0] = max(0.0, args.settle_ms)
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(each GPU would run its own share of sequences/heads independently).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import gated_delta_rule_44_amd as gdr
    from gated_delta_rule_44_amd import synthetic
    dev = torch.device("cuda:0")

    if args.only == "gdn_prefill":
        ms = bench_prefill(gdr, synthetic, torch, dev, 4, 4096, 16, "scalar", 1001,
                           args.steps, args.warmup)
        print(json.dumps({"workload": "gdn_prefill_B4_H16_T4096_d128_bf16", "ms_per_step": ms,
                          "ms_per_step_mean": LAST_MEAN_MS[0]}))
        return
    if args.only == "recurrent":
        ms = bench_recurrent(gdr, synthetic, torch, dev, args.steps, args.warmup)
        print(json.dumps({"workload": "gdn_recurrent_B1_H1_T64_d64_fp32", "latency_us": ms * 1e3}))
        return
    if args.only == "hbm_copy":
        # a plain device-to-device copy of 1 GiB: what the memory system
        # reaches for a pure stream, and the known byte count that the HBM
        # counters are calibrated against
        src = torch.empty(1 << 28, device=dev, dtype=torch.float32).normal_()
        dst = torch.empty_like(src)
        ms = timed(lambda i: dst.copy_(src), args.steps, args.warmup, torch.cuda.current_stream(dev))
        nb = 2 * src.numel() * 4
        print(json.dumps({"workload": "hbm_copy_1GiB", "ms_per_step": ms, "bytes_per_step": nb,
                          "GB_per_s": nb / (ms * 1e-3) / 1e9, "frac_hbm": nb / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}))
        return
    if args.only == "kda_prefill":
        ms = bench_prefill(gdr, synthetic, torch, dev, 2, 8192, 32, "channel", 1002,
                           args.steps, args.warmup, h0=False)
        print(json.dumps({"workload": "kda_prefill_B2_H32_T8192_d128_bf16", "ms_per_step": ms}))
        return
    if args.only == "decode":
        ms, _, _, _ = bench_decode(gdr, synthetic, torch, dev, args.steps, args.warmup)
        print(json.dumps({"workload": "placement_decode_L48_B256_H32_d128_bf16", "ms_per_step": ms}))
        return
    if args.only == "varlen":
        ms, _, _ = bench_varlen(gdr, synthetic, torch, dev, args.steps, args.warmup)
        print(json.dumps({"workload": "kda_varlen_N16_H32_d128_bf16", "ms_per_step": ms}))
        return
    if args.only in ("fused_gdn", "fused_kda"):
        if args.only == "fused_gdn":
            ms = bench_fused(gdr, synthetic, torch, dev, 4, 4096, 16, "scalar", 1011,
                             args.steps, args.warmup)
            name = "fused_gdn_prefill_B4_H16_T4096_d128_bf16"
        else:
            ms = bench_fused(gdr, synthetic, torch, dev, 2, 8192, 32, "channel", 1012,
                             args.steps, args.warmup, h0=False)
            name = "fused_kda_prefill_B2_H32_T8192_d128_bf16"
        print(json.dumps({"workload": name, "ms_per_step": ms}))
        return
    if args.only in ("backward_gdn", "backward_kda"):
        if args.only == "backward_gdn":
            ms = bench_backward(gdr, synthetic, torch, dev, 4, 4096, 16, "scalar", 1001,
                                args.steps, args.warmup)
            name = "backward_gdn_B4_H16_T4096_d128_bf16"
        else:
            ms = bench_backward(gdr, synthetic, torch, dev, 2, 8192, 32, "channel", 1002,
                                args.steps, args.warmup, h0=False)
            name = "backward_kda_B2_H32_T8192_d128_bf16"
        print(json.dumps({"workload": name, "ms_per_step": ms}))
        return
    if args.only == "backward_kda_varlen":
        ms, _, _ = bench_backward_varlen(gdr, synthetic, torch, dev, args.steps, args.warmup)
        print(json.dumps({"workload": "backward_kda_varlen_N16_H32_d128_bf16", "ms_per_step": ms}))
        return
    if args.only == "draft":
        md, mc, _, _, _, _ = bench_draft(gdr, synthetic, torch, dev, args.steps, args.warmup)
        print(json.dumps({"workload": "gdn_draft_decode_B256_n4_H32_d128_bf16",
                          "ms_draft": md, "ms_commit": mc}))
        return
    if args.only == "varlen_pool":
        ms, _ = bench_varlen_pool(gdr, synthetic, torch, dev, args.steps, args.warmup)
        print(json.dumps({"workload": "kda_varlen_pool_N16_H32_d128_bf16", "ms_per_step": ms}))
        return

    B, T, H = 4, 4096, 16
    ms = bench_prefill(gdr, synthetic, torch, dev, B, T, H, "scalar", 1001,
                       args.steps, args.warmup)
    ms_mean = LAST_MEAN_MS[0]
    settle_calls = LAST_SETTLE_CALLS[0]
    tokens = B * T
    th = tokens * H
    nbytes = prefill_bytes(th, B * H, "scalar")
    flops = prefill_flops(th)
    # the roofline takes the average call time (the rocprofv3 kernel
    # averages are averages too); value and ms_per_step the median
    achieved = nbytes / (ms_mean * 1e-3) / 1e9
    line = {
        "metric": METRIC,
        "value": tokens / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "clock_settle_calls": settle_calls,
        "ms_per_step": ms,
        "ms_per_step_mean": ms_mean,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "gdn_prefill_B4_H16_T4096_d128_bf16", "B": B, "T": T,
                   "H": H, "d_k": D, "d_v": D, "chunk": C, "gate": "scalar (GDN)",
                   "state": "fp32, h0 and ht", "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": (measured_traffic("gdn_prefill") or {}).get("bytes_per_call"),
                     "kernel": "prep_kernel<128> + chain_kernel<128> (one gdr_prefill_chunked call)",
                     "algorithmic_bytes_per_launch": nbytes,
                     "mfma_tflops_alg": flops / (ms_mean * 1e-3) / 1e12,
                     "mfma_frac_alg": flops / (ms_mean * 1e-3) / 1e12 / MFMA_BF16_TFLOPS},
    }

    if not args.only_headline:
        sec = []
        # the fp32 recurrent GDN workload (B=1 H=1 T=64 d=64): the latency of
        # one call
        ms0 = bench_recurrent(gdr, synthetic, torch, dev, args.steps, args.warmup)
        sec.append({"workload": "gdn_recurrent_B1_H1_T64_d64_fp32", "latency_us": ms0 * 1e3,
                    "latency_us_mean": LAST_MEAN_MS[0] * 1e3,
                    "tokens_per_s": 64 / (ms0 * 1e-3)})
        ms2 = bench_prefill(gdr, synthetic, torch, dev, 2, 8192, 32, "channel", 1002,
                            args.steps, args.warmup, h0=False, sets=3)
        th2 = 2 * 8192 * 32
        b2 = prefill_bytes(th2, 64, "channel") - 64 * D * D * 4   # no h0 read
        sec.append({"workload": "kda_prefill_B2_H32_T8192_d128_bf16",
                    "ms_per_step": ms2, "tokens_per_s": 2 * 8192 / (ms2 * 1e-3),
                    "GB_per_s": b2 / (ms2 * 1e-3) / 1e9,
                    "frac_hbm": b2 / (ms2 * 1e-3) / 1e9 / HBM_PEAK_GBS,
                    "mfma_frac_alg": prefill_flops(th2) / (ms2 * 1e-3) / 1e12 / MFMA_BF16_TFLOPS})
        ms3, n_gdn, n_kda, pstr = bench_decode(gdr, synthetic, torch, dev,
                                               max(5, args.steps // 5), max(2, args.warmup // 5))
        hs = (n_gdn + n_kda) * 256 * 32
        b3 = decode_bytes(hs, (n_gdn * 4 + n_kda * 4 * D) * 256 * 32)
        sec.append({"workload": "placement_decode_L48_B256_H32_d128_bf16",
                    "placement": pstr, "recurrent_layers": n_gdn + n_kda,
                    "ms_per_step": ms3, "tokens_per_s": 256 / (ms3 * 1e-3),
                    "GB_per_s": b3 / (ms3 * 1e-3) / 1e9,
                    "frac_hbm": b3 / (ms3 * 1e-3) / 1e9 / HBM_PEAK_GBS})
        ms4, tok4, lens = bench_varlen(gdr, synthetic, torch, dev,
                                       max(5, args.steps // 5), max(2, args.warmup // 5))
        b4 = prefill_bytes(tok4 * 32, 16 * 32, "channel")
        sec.append({"workload": "kda_varlen_N16_H32_d128_bf16", "tokens": tok4,
                    "ms_per_step": ms4, "tokens_per_s": tok4 / (ms4 * 1e-3),
                    "GB_per_s": b4 / (ms4 * 1e-3) / 1e9,
                    "frac_hbm": b4 / (ms4 * 1e-3) / 1e9 / HBM_PEAK_GBS,
                    "mfma_frac_alg": prefill_flops(tok4 * 32) / (ms4 * 1e-3) / 1e12 / MFMA_BF16_TFLOPS})
        md, mc, Bd, nd, Hd, kept = bench_draft(gdr, synthetic, torch, dev,
                                               max(5, args.steps // 5), max(2, args.warmup // 5))
        state = D * D * 4
        bd = Bd * Hd * ((1 + nd) * state + nd * (3 * D * 2 + D * 2 + 4 + 4))
        bc = kept * Hd * 2 * state
        sec.append({"workload": "gdn_draft_decode_B256_n4_H32_d128_bf16",
                    "pool_slots": 512, "draft_tokens": nd,
                    "ms_draft": md, "draft_GB_per_s": bd / (md * 1e-3) / 1e9,
                    "draft_frac_hbm": bd / (md * 1e-3) / 1e9 / HBM_PEAK_GBS,
                    "draft_tokens_per_s": Bd * nd / (md * 1e-3),
                    "ms_commit": mc, "commit_GB_per_s": bc / (mc * 1e-3) / 1e9,
                    "commit_frac_hbm": bc / (mc * 1e-3) / 1e9 / HBM_PEAK_GBS})
        ms6, tok6 = bench_varlen_pool(gdr, synthetic, torch, dev,
                                      max(5, args.steps // 5), max(2, args.warmup // 5))
        b6 = prefill_bytes(tok6 * 32, 16 * 32, "channel")
        sec.append({"workload": "kda_varlen_pool_N16_H32_d128_bf16", "pool_slots": 40,
                    "ms_per_step": ms6, "tokens_per_s": tok6 / (ms6 * 1e-3),
                    "GB_per_s": b6 / (ms6 * 1e-3) / 1e9,
                    "frac_hbm": b6 / (ms6 * 1e-3) / 1e9 / HBM_PEAK_GBS})
        # fused preprocessing: raw bf16 projections and logits (gate 2 B per
        # value instead of 4), q/k normalised in the kernels
        for gate, B_, T_, H_, seed, h0_, name in (
                ("scalar", 4, 4096, 16, 1011, True, "fused_gdn_prefill_B4_H16_T4096_d128_bf16"),
                ("channel", 2, 8192, 32, 1012, False, "fused_kda_prefill_B2_H32_T8192_d128_bf16")):
            msf = bench_fused(gdr, synthetic, torch, dev, B_, T_, H_, gate, seed,
                              args.steps, args.warmup, h0=h0_)
            thf = B_ * T_ * H_
            per_tok = 3 * D * 2 + D * 2 + 2 + (2 * D if gate == "channel" else 2)
            bf = thf * per_tok + B_ * H_ * (2 if h0_ else 1) * D * D * 4
            sec.append({"workload": name, "ms_per_step": msf,
                        "tokens_per_s": B_ * T_ / (msf * 1e-3),
                        "GB_per_s": bf / (msf * 1e-3) / 1e9,
                        "frac_hbm": bf / (msf * 1e-3) / 1e9 / HBM_PEAK_GBS,
                        "mfma_frac_alg": prefill_flops(thf) / (msf * 1e-3) / 1e12 / MFMA_BF16_TFLOPS})
        # backward of the two prefill workloads
        for gate, B_, T_, H_, seed, h0_, name in (
                ("scalar", 4, 4096, 16, 1001, True, "backward_gdn_B4_H16_T4096_d128_bf16"),
                ("channel", 2, 8192, 32, 1002, False, "backward_kda_B2_H32_T8192_d128_bf16")):
            msb = bench_backward(gdr, synthetic, torch, dev, B_, T_, H_, gate, seed,
                                 max(5, args.steps // 5), max(2, args.warmup // 5), h0=h0_)
            bb = backward_bytes(B_ * T_ * H_, B_ * H_, gate, h0_)
            sec.append({"workload": name, "ms_per_step": msb,
                        "tokens_per_s": B_ * T_ / (msb * 1e-3),
                        "GB_per_s": bb / (msb * 1e-3) / 1e9,
                        "frac_hbm": bb / (msb * 1e-3) / 1e9 / HBM_PEAK_GBS})
        # the same GDN backward with g = -4 per token everywhere: every
        # (sequence, head) has chunks decaying by e^-256 and takes the exact
        # token-level path
        msw = bench_backward(gdr, synthetic, torch, dev, 4, 4096, 16, "scalar", 1001,
                             max(3, args.steps // 10), max(1, args.warmup // 10), gate_fill=-4.0)
        bb = backward_bytes(4 * 4096 * 16, 64, "scalar", True)
        sec.append({"workload": "backward_gdn_B4_H16_T4096_d128_bf16_all_pairs_past_chunk_range",
                    "gate": "g = -4 per token (every pair on the token-level path)",
                    "ms_per_step": msw, "tokens_per_s": 4 * 4096 / (msw * 1e-3),
                    "GB_per_s": bb / (msw * 1e-3) / 1e9,
                    "frac_hbm": bb / (msw * 1e-3) / 1e9 / HBM_PEAK_GBS})
        msv, tokv, nv = bench_backward_varlen(gdr, synthetic, torch, dev,
                                              max(3, args.steps // 40), max(1, args.warmup // 50))
        bb = backward_bytes(tokv * 32, nv * 32, "channel", True)
        sec.append({"workload": "backward_kda_varlen_N16_H32_d128_bf16", "tokens": tokv,
                    "ms_per_step": msv, "tokens_per_s": tokv / (msv * 1e-3),
                    "GB_per_s": bb / (msv * 1e-3) / 1e9,
                    "frac_hbm": bb / (msv * 1e-3) / 1e9 / HBM_PEAK_GBS})
        keys = {"kda_prefill_B2_H32_T8192_d128_bf16": "kda_prefill",
                "placement_decode_L48_B256_H32_d128_bf16": "decode",
                "kda_varlen_N16_H32_d128_bf16": "varlen",
                "gdn_draft_decode_B256_n4_H32_d128_bf16": "draft",
                "fused_gdn_prefill_B4_H16_T4096_d128_bf16": "fused_gdn",
                "fused_kda_prefill_B2_H32_T8192_d128_bf16": "fused_kda",
                "backward_gdn_B4_H16_T4096_d128_bf16": "backward_gdn",
                "backward_kda_B2_H32_T8192_d128_bf16": "backward_kda",
                "gdn_recurrent_B1_H1_T64_d64_fp32": "recurrent",
                "kda_varlen_pool_N16_H32_d128_bf16": "varlen_pool",
                "backward_kda_varlen_N16_H32_d128_bf16": "backward_kda_varlen"}
        for e in sec:
            if e["workload"] in keys:
                e["traffic"] = measured_traffic(keys[e["workload"]])
        line["secondary"] = sec

    if not args.no_cpu_baseline:
        head, others = cpu_baseline(synthetic, torch)
        line["cpu_baseline"] = head
        for e in others:
            for s_ in line.get("secondary", []):
                if s_["workload"] == e["workload"]:
                    s_["cpu_baseline"] = {k: v for k, v in e.items() if k != "workload"}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
