"""Seeded synthetic inputs for the gated delta rule.

This module only draws random numbers and lays them out; it holds none of
the recurrence's arithmetic.  Both the HIP path (through the binding) and the
CPU oracle consume what it produces, always the *stored* values.

Recipe (one generator per call, drawn in this fixed order: q, k, v,
beta-logit, gate-logit, h0):
  * q, k : N(0,1) in fp32, divided by their per-token L2 norm, then cast to
           the input dtype (the kernels never normalise; the oracle consumes
           the rounded values).
  * v    : N(0,1), cast.
  * beta : sigmoid(N(0,1)), fp32, one per (token, head).
  * g    : log-gate g = ln a = -softplus(N(0,1)) * c, fp32; [.., H] for a
           scalar (Gated DeltaNet) gate with c = 0.1, [.., H, Dk] for a
           per-channel (Kimi Delta Attention) gate with c = 0.05.
  * h0   : 0.02 * N(0,1) fp32 (N(0, 0.02) read as standard deviation), or
           None for a zero initial state.

The mixer set {full attention, sliding window, KDA, GDN} and the one mixer
per layer placement come from "Super Apriel: One Checkpoint, Many Speeds"
(abstract; gist.science summary section 2a).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

FA, SWA, GDN, KDA = 0, 1, 2, 3
MIXER_NAMES = "FSGK"
GATE_SCALE = {"scalar": 0.1, "channel": 0.05}


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _unit_rows(shape, gen, device, dtype):
    x = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    x = x / x.norm(dim=-1, keepdim=True)
    return x.to(dtype)


def _draw(shape_tok, H, Dk, Dv, dtype, gate, gen, device, h0_shape=None,
          gate_scale=None):
    """shape_tok: leading token dims, e.g. (B, T) or (T_total,)."""
    q = _unit_rows((*shape_tok, H, Dk), gen, device, dtype)
    k = _unit_rows((*shape_tok, H, Dk), gen, device, dtype)
    v = torch.randn((*shape_tok, H, Dv), generator=gen, device=device,
                    dtype=torch.float32).to(dtype)
    beta = torch.sigmoid(torch.randn((*shape_tok, H), generator=gen,
                                     device=device, dtype=torch.float32))
    c = GATE_SCALE[gate] if gate_scale is None else gate_scale
    gshape = (*shape_tok, H, Dk) if gate == "channel" else (*shape_tok, H)
    g = -torch.nn.functional.softplus(
        torch.randn(gshape, generator=gen, device=device,
                    dtype=torch.float32)) * c
    h0 = None
    if h0_shape is not None:
        h0 = torch.randn(h0_shape, generator=gen, device=device,
                         dtype=torch.float32) * 0.02
    return dict(q=q.contiguous(), k=k.contiguous(), v=v.contiguous(),
                g=g.contiguous(), beta=beta.contiguous(), h0=h0)


def prefill_inputs(B, T, H, D, dtype=torch.bfloat16, gate="scalar", seed=0,
                   h0=True, device="cpu", Dv=None, gate_scale=None):
    """Fixed-length batch: q,k [B,T,H,D], v [B,T,H,Dv], g [B,T,H](,D),
    beta [B,T,H], h0 [B,H,Dv,D] or None."""
    Dv = D if Dv is None else Dv
    gen = _gen(seed, device)
    return _draw((B, T), H, D, Dv, dtype, gate, gen, device,
                 h0_shape=(B, H, Dv, D) if h0 else None, gate_scale=gate_scale)


def varlen_lengths(seed=943, n=16, lo=512, hi=65536):
    """Sequence lengths drawn log-uniform on [lo, hi] with numpy's PCG64."""
    rng = np.random.default_rng(seed)
    return [int(x) for x in
            np.floor(np.exp(rng.uniform(np.log(lo), np.log(hi), n)))]


def cu_from_lengths(lengths):
    return np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)


def varlen_inputs(lengths, H, D, dtype=torch.bfloat16, gate="channel", seed=0,
                  h0=True, device="cpu", gate_scale=None):
    """Packed batch: q,k [T_tot,H,D] ..., cu_seqlens int32 [N+1] (on device and
    as a host numpy copy), h0 [N,H,D,D] or None."""
    cu = cu_from_lengths(lengths)
    gen = _gen(seed, device)
    d = _draw((int(cu[-1]),), H, D, D, dtype, gate, gen, device,
              h0_shape=(len(lengths), H, D, D) if h0 else None,
              gate_scale=gate_scale)
    d["cu_seqlens"] = torch.from_numpy(cu).to(device)
    d["cu_seqlens_host"] = cu
    return d


def placement(seed=0, n_layers=48):
    """Balanced placement: equal counts of FA/SWA/GDN/KDA, permuted by
    numpy's PCG64 with the given seed.  Returns a uint8 numpy array."""
    per = n_layers // 4
    rng = np.random.default_rng(seed)
    return rng.permutation(np.repeat(np.arange(4), per)).astype(np.uint8)


def placement_string(p):
    return "".join(MIXER_NAMES[int(x)] for x in p)


def decode_inputs(L, B, H, D, dtype=torch.bfloat16, place=None, seed=0,
                  device="cpu", pool=True):
    """Placement decode batch.  q,k [L,B,H,D], v [L,B,H,D], g [L,B,H,D]
    (layers tagged GDN use channel 0 only, drawn with the scalar-gate scale;
    KDA layers with the channel scale), beta [L,B,H], pool [L,B,H,D,D] fp32
    0.02*N(0,1).  Every layer slot is drawn, whatever its mixer, so that the
    untouched slots hold ordinary values."""
    place = placement(0, L) if place is None else np.asarray(place, np.uint8)
    gen = _gen(seed, device)
    q = _unit_rows((L, B, H, D), gen, device, dtype).contiguous()
    k = _unit_rows((L, B, H, D), gen, device, dtype).contiguous()
    v = torch.randn((L, B, H, D), generator=gen, device=device,
                    dtype=torch.float32).to(dtype).contiguous()
    beta = torch.sigmoid(torch.randn((L, B, H), generator=gen, device=device,
                                     dtype=torch.float32)).contiguous()
    g = torch.empty((L, B, H, D), device=device, dtype=torch.float32)
    for layer in range(L):
        c = GATE_SCALE["scalar"] if place[layer] == GDN else GATE_SCALE["channel"]
        x = torch.randn((B, H, D), generator=gen, device=device,
                        dtype=torch.float32)
        g[layer] = -torch.nn.functional.softplus(x) * c
    st = None
    if pool:
        st = torch.empty((L, B, H, D, D), device=device, dtype=torch.float32)
        for layer in range(L):
            st[layer].normal_(0.0, 0.02, generator=gen)
    return dict(q=q, k=k, v=v, g=g, beta=beta, pool=st, placement=place)


def _draw_raw(shape_tok, H, D, dtype, gate, gen, device, h0_shape=None):
    """Raw projections: q, k, v ~ N(0,1) (q and k not normalised), beta and
    gate logits ~ N(0,1), all stored in dtype; h0 0.02 N(0,1) fp32."""
    q = torch.randn((*shape_tok, H, D), generator=gen, device=device).to(dtype)
    k = torch.randn((*shape_tok, H, D), generator=gen, device=device).to(dtype)
    v = torch.randn((*shape_tok, H, D), generator=gen, device=device).to(dtype)
    xb = torch.randn((*shape_tok, H), generator=gen, device=device).to(dtype)
    gshape = (*shape_tok, H, D) if gate == "channel" else (*shape_tok, H)
    xg = torch.randn(gshape, generator=gen, device=device).to(dtype)
    h0 = None
    if h0_shape is not None:
        h0 = torch.randn(h0_shape, generator=gen, device=device, dtype=torch.float32) * 0.02
    return dict(q=q.contiguous(), k=k.contiguous(), v=v.contiguous(),
                gate_logit=xg.contiguous(), beta_logit=xb.contiguous(), h0=h0,
                gate_scale=GATE_SCALE[gate])


def raw_prefill_inputs(B, T, H, D, dtype=torch.bfloat16, gate="scalar", seed=0,
                       h0=True, device="cpu"):
    """Fixed-length batch of raw projections for the fused-preprocessing
    calls: q, k, v [B,T,H,D], gate_logit [B,T,H](,D), beta_logit [B,T,H],
    all in dtype, h0 [B,H,D,D] fp32 or None, and the gate scale c."""
    return _draw_raw((B, T), H, D, dtype, gate, _gen(seed, device), device,
                     h0_shape=(B, H, D, D) if h0 else None)


def raw_varlen_inputs(lengths, H, D, dtype=torch.bfloat16, gate="channel", seed=0,
                      h0=True, device="cpu"):
    """Packed batch of raw projections (as raw_prefill_inputs) with
    cu_seqlens on the device and as a host numpy copy."""
    cu = cu_from_lengths(lengths)
    d = _draw_raw((int(cu[-1]),), H, D, dtype, gate, _gen(seed, device), device,
                  h0_shape=(len(lengths), H, D, D) if h0 else None)
    d["cu_seqlens"] = torch.from_numpy(cu).to(device)
    d["cu_seqlens_host"] = cu
    return d


def pool_states(P, H, D, seed=0, device="cpu"):
    """A state pool [P,H,D,D] fp32 with 0.02*N(0,1) entries (the law of the
    initial states), drawn slot by slot."""
    gen = _gen(seed, device)
    st = torch.empty((P, H, D, D), device=device, dtype=torch.float32)
    for p in range(P):
        st[p].normal_(0.0, 0.02, generator=gen)
    return st


def serving_slots(B, P, idle=0, seed=0):
    """Distinct pool slots for B sequences (a seeded draw from 0..P-1 with
    numpy's PCG64), `idle` of them replaced by -1.  int32 numpy array."""
    rng = np.random.default_rng(seed)
    s = rng.permutation(P)[:B].astype(np.int32)
    if idle:
        s[rng.choice(B, idle, replace=False)] = -1
    return s


def accepted_counts(B, n, seed=0):
    """Accepted prefix length of each sequence's n drafted tokens, uniform
    on 0..n (numpy's PCG64).  int32 numpy array."""
    return np.random.default_rng(seed).integers(0, n + 1, B).astype(np.int32)


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str          # "prefill" | "decode" | "varlen"
    gate: str          # "scalar" | "channel" | "placement"
    dtype: torch.dtype
    B: int = 1
    T: int = 0
    H: int = 1
    D: int = 128
    L: int = 0
    h0: bool = False
    seed: int = 0


# The five synthetic workloads (seed = 1000 + index).
WORKLOADS = [
    Workload("gdn_recurrent_B1_H1_T64_d64_fp32", "prefill", "scalar",
             torch.float32, B=1, T=64, H=1, D=64, h0=False, seed=1000),
    Workload("gdn_prefill_B4_H16_T4096_d128_bf16", "prefill", "scalar",
             torch.bfloat16, B=4, T=4096, H=16, D=128, h0=True, seed=1001),
    Workload("kda_prefill_B2_H32_T8192_d128_bf16", "prefill", "channel",
             torch.bfloat16, B=2, T=8192, H=32, D=128, h0=False, seed=1002),
    Workload("placement_decode_L48_B256_H32_d128_bf16", "decode", "placement",
             torch.bfloat16, B=256, H=32, D=128, L=48, h0=True, seed=1003),
    Workload("kda_varlen_N16_H32_d128_bf16", "varlen", "channel",
             torch.bfloat16, H=32, D=128, h0=True, seed=1004),
]
