"""fp64 CPU oracle for the gated delta rule -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product package
(``gated_delta_rule_44_amd``) never imports it, and the two share no code.

The arithmetic lives in ``gdr_oracle.c`` (plain C, fp64, one token at a time,
built with gcc).  This module only builds/loads that library and marshals
arrays: it widens the *stored* input values (bf16 or fp32) to float32, which
is exact, and hands them over.

Source of the method: "Super Apriel: One Checkpoint, Many Speeds"
(arXiv 2604.19877).  Its gist.science technical summary, section 2a, lists
Kimi Delta Attention as recurrent with a per-channel gate and Gated DeltaNet
as recurrent with a scalar gate; the recurrence itself is the standard gated
delta rule stated in ``gdr_oracle.c``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdr_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(src: str = _SRC, out: str = _LIB, extra_flags=()) -> str:
    """Compile the oracle with gcc (-O2, OpenMP) into a shared library."""
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-fopenmp",
           *extra_flags, src, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def _bind(lib):
    f = lib.gdr_oracle_forward
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                  ctypes.c_int, ctypes.c_int, ctypes.c_double,
                  ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                  ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                  ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int]
    b = lib.gdr_oracle_backward
    b.restype = ctypes.c_int
    b.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                  ctypes.c_int, ctypes.c_int, ctypes.c_double] + [ctypes.c_void_p] * 14 + [
                  ctypes.c_int]
    lib.gdr_oracle_max_threads.restype = ctypes.c_int
    return lib


def load(path: str | None = None):
    """Load (building first if absent) the oracle library."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(path))
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        _lib = _bind(ctypes.CDLL(_LIB))
    return _lib


def _f32(x) -> np.ndarray:
    """Stored values -> contiguous float32 ndarray (exact for bf16/fp32)."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().to("cpu")
            if x.dtype != torch.float32:
                x = x.to(torch.float32)
            return np.ascontiguousarray(x.numpy())
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(x, dtype=np.float32))


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def forward(q, k, v, g, beta, h0=None, cu_seqlens=None, scale: float = 1.0,
            threads: int | None = None, lib=None):
    """Gated delta rule over a batch, token by token in fp64.

    Layouts (row-major):
      fixed batch : q,k [B,T,H,Dk]  v [B,T,H,Dv]  g [B,T,H] or [B,T,H,Dk]
                    beta [B,T,H]    h0 [B,H,Dv,Dk] or None
      packed      : (cu_seqlens given, int [N+1]) q,k [T_tot,H,Dk] ...,
                    h0 [N,H,Dv,Dk] or None
    A gate with as many dims as q is a per-channel gate; one dim fewer is a
    scalar (per token and head) gate.  Returns (o, ht) as float64 arrays with
    o shaped like v and ht [N,H,Dv,Dk].
    """
    lib = lib or load()
    qf, kf, vf, gf, bf = (_f32(x) for x in (q, k, v, g, beta))
    channel = gf.ndim == qf.ndim
    if cu_seqlens is None:
        B, T, H, Dk = qf.shape
        cu = np.arange(B + 1, dtype=np.int64) * T
    else:
        cu = np.ascontiguousarray(np.asarray(
            cu_seqlens.cpu() if hasattr(cu_seqlens, "cpu") else cu_seqlens,
            dtype=np.int64))
        _, H, Dk = qf.shape
    Dv = vf.shape[-1]
    N = len(cu) - 1
    hf = None if h0 is None else _f32(h0)
    o = np.zeros(vf.shape, dtype=np.float64)
    ht = np.zeros((N, H, Dv, Dk), dtype=np.float64)
    rc = lib.gdr_oracle_forward(
        N, _ptr(cu), H, Dk, Dv, int(channel), float(scale),
        _ptr(qf), _ptr(kf), _ptr(vf), _ptr(gf), _ptr(bf), _ptr(hf),
        _ptr(o), _ptr(ht), int(threads or 0))
    if rc != 0:
        raise RuntimeError("gdr_oracle_forward failed with code %d" % rc)
    return o, ht


def backward_c(q, k, v, g, beta, do, h0=None, dht=None, cu_seqlens=None,
               scale: float = 1.0, threads: int | None = None, lib=None):
    """Gradients (dq, dk, dv, dg, dbeta, dh0) of sum(o * do) + sum(S_T * dht)
    by the C oracle's hand-written fp64 vector-Jacobian product (one token at
    a time, states recomputed from checkpoints), for the large cases the
    autograd form ``backward`` cannot hold in memory.  Layouts as
    ``forward`` (fixed or packed); do like v, dht like h0.  Float64 arrays
    shaped like q, k, v, g, beta and [N, H, Dv, Dk]."""
    lib = lib or load()
    qf, kf, vf, gf, bf, df = (_f32(x) for x in (q, k, v, g, beta, do))
    channel = gf.ndim == qf.ndim
    if cu_seqlens is None:
        B, T, H, Dk = qf.shape
        cu = np.arange(B + 1, dtype=np.int64) * T
    else:
        cu = np.ascontiguousarray(np.asarray(
            cu_seqlens.cpu() if hasattr(cu_seqlens, "cpu") else cu_seqlens,
            dtype=np.int64))
        _, H, Dk = qf.shape
    Dv = vf.shape[-1]
    N = len(cu) - 1
    hf = None if h0 is None else _f32(h0)
    dtf = None if dht is None else _f32(dht)
    out = [np.zeros(x.shape, dtype=np.float64) for x in (qf, kf, vf, gf, bf)]
    dh0 = np.zeros((N, H, Dv, Dk), dtype=np.float64)
    rc = lib.gdr_oracle_backward(
        N, _ptr(cu), H, Dk, Dv, int(channel), float(scale),
        _ptr(qf), _ptr(kf), _ptr(vf), _ptr(gf), _ptr(bf), _ptr(hf), _ptr(df), _ptr(dtf),
        *(_ptr(x) for x in out), _ptr(dh0), int(threads or 0))
    if rc != 0:
        raise RuntimeError("gdr_oracle_backward failed with code %d" % rc)
    return tuple(out) + (dh0,)


def decode(q, k, v, g, beta, state, scale: float = 1.0, threads=None, lib=None):
    """One decode step per (b, h): q,k [B,H,Dk], v [B,H,Dv], g [B,H] or
    [B,H,Dk], beta [B,H], state [B,H,Dv,Dk].  Returns (o [B,H,Dv], new state),
    both float64.  This is the same recurrence over a length-1 sequence."""
    qf = _f32(q)
    B, H, Dk = qf.shape
    add_t = lambda x: _f32(x)[:, None]  # noqa: E731  [B,1,...]
    o, ht = forward(add_t(q), add_t(k), add_t(v), add_t(g), add_t(beta),
                    h0=state, scale=scale, threads=threads, lib=lib)
    return o[:, 0], ht


def max_threads(lib=None) -> int:
    return (lib or load()).gdr_oracle_max_threads()


def _slot_ok(s, pool):
    return 0 <= int(s) < pool


def decode_tokens(q, k, v, g, beta, state_pool, slot=None, checkpoints=False,
                  scale: float = 1.0, threads=None, lib=None):
    """n decode tokens for each of B sequences whose states live in a pool.

    q,k [B,n,H,Dk], v [B,n,H,Dv], g [B,n,H] or [B,n,H,Dk], beta [B,n,H],
    state_pool [P,H,Dv,Dk], slot [B] (None: slot b; a value outside 0..P-1
    marks an idle sequence).  Written out from the definition: the state of
    each active sequence is gathered from its slot, the recurrence runs over
    its n tokens (``forward``), and the final state is scattered back -- or,
    with checkpoints, the state after token t is the final state of the
    recurrence over tokens 0..t (one ``forward`` per prefix) and the pool is
    left as it was.  Returns (o [B,n,H,Dv] with NaN rows for idle sequences,
    new pool [P,H,Dv,Dk], checkpoints [B,n,H,Dv,Dk] or None), all float64.
    """
    qf, kf, vf, gf, bf = (_f32(x) for x in (q, k, v, g, beta))
    pool = _f32(state_pool)
    B, n = qf.shape[:2]
    P = pool.shape[0]
    slots = np.arange(B) if slot is None else np.asarray(
        slot.cpu() if hasattr(slot, "cpu") else slot, dtype=np.int64)
    act = np.array([b for b in range(B) if _slot_ok(slots[b], P)], dtype=np.int64)
    o = np.full(vf.shape, np.nan)
    new_pool = pool.astype(np.float64)
    ck = None
    if checkpoints:
        ck = np.full((B, n) + pool.shape[1:], np.nan)
    if len(act) == 0 or n == 0:
        return o, new_pool, ck
    h0 = pool[slots[act]]
    sel = lambda x: x[act]  # noqa: E731
    o_a, ht = forward(sel(qf), sel(kf), sel(vf), sel(gf), sel(bf), h0=h0,
                      scale=scale, threads=threads, lib=lib)
    o[act] = o_a
    if checkpoints:
        for t in range(n):
            pre = lambda x: np.ascontiguousarray(x[act, :t + 1])  # noqa: E731
            _, st = forward(pre(qf), pre(kf), pre(vf), pre(gf), pre(bf), h0=h0,
                            scale=scale, threads=threads, lib=lib)
            ck[act, t] = st
    else:
        new_pool[slots[act]] = ht
    return o, new_pool, ck


def forward_pool(q, k, v, g, beta, cu_seqlens, state_pool, h0_slot, ht_slot,
                 scale: float = 1.0, threads=None, lib=None):
    """Packed-batch recurrence with initial and final states in a pool.

    Sequence n starts from state_pool[h0_slot[n]] (zeros when the slot is
    outside 0..P-1) and its final state is written to state_pool[ht_slot[n]]
    (nothing when outside).  Gather, ``forward``, scatter.  Returns
    (o [T_tot,H,Dv], new pool [P,H,Dv,Dk]) as float64.
    """
    pool = _f32(state_pool)
    P = pool.shape[0]
    to_np = lambda x: np.asarray(x.cpu() if hasattr(x, "cpu") else x, dtype=np.int64)  # noqa: E731
    s0, s1 = to_np(h0_slot), to_np(ht_slot)
    N = len(s0)
    h0 = np.zeros((N,) + pool.shape[1:], dtype=np.float32)
    for i in range(N):
        if _slot_ok(s0[i], P):
            h0[i] = pool[s0[i]]
    o, ht = forward(q, k, v, g, beta, h0=h0, cu_seqlens=cu_seqlens, scale=scale,
                    threads=threads, lib=lib)
    new_pool = pool.astype(np.float64)
    for i in range(N):
        if _slot_ok(s1[i], P):
            new_pool[s1[i]] = ht[i]
    return o, new_pool


# Fused input preprocessing.  The kernels can take the projections as they
# come out of a layer: q and k un-normalised, and logits for beta and the
# gate.  The definitions, in fp64:
#     q_hat = q / sqrt(|q|^2 + NORM_EPS)        (per token and head)
#     beta  = 1 / (1 + e^{-x_beta})
#     g     = -c * softplus(x_g) = -c * ln(1 + e^{x_g})
NORM_EPS = 1e-6


def _f64(x):
    return _f32(x).astype(np.float64)


def preprocess(q, k, gate_logit, beta_logit, gate_scale: float):
    """Raw projections -> (q_hat, k_hat, g, beta) as float32 arrays.

    The fp64 results are rounded once to float32, the width the recurrence
    oracle reads (a relative change below 2^-24)."""
    qf, kf, xg, xb = (_f64(x) for x in (q, k, gate_logit, beta_logit))
    qh = qf / np.sqrt((qf * qf).sum(-1, keepdims=True) + NORM_EPS)
    kh = kf / np.sqrt((kf * kf).sum(-1, keepdims=True) + NORM_EPS)
    beta = 1.0 / (1.0 + np.exp(-xb))
    # ln(1 + e^x) without overflow: max(x, 0) + ln(1 + e^{-|x|})
    softplus = np.maximum(xg, 0.0) + np.log1p(np.exp(-np.abs(xg)))
    g = -float(gate_scale) * softplus
    return tuple(np.ascontiguousarray(a.astype(np.float32)) for a in (qh, kh, g, beta))


# --------------------------------------------------------------------------
# Backward: the vector-Jacobian product of the recurrence.  Written out as
# the forward recurrence in plain PyTorch CPU ops in fp64 (token by token,
# the same steps as gdr_oracle.c) and differentiated by autograd: for
# upstream gradients dO (of o) and dht (of the final state), it returns the
# gradients of L = sum(o * dO) + sum(S_T * dht).

def forward_torch(q, k, v, g, beta, h0=None, scale: float = 1.0):
    """The recurrence on float64 torch tensors (fixed-length batch layouts
    as ``forward``), differentiable.  Returns (o, S_T)."""
    import torch
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    channel = g.dim() == q.dim()
    S = (torch.zeros((B, H, Dv, Dk), dtype=torch.float64) if h0 is None else h0)
    outs = []
    for t in range(T):
        a = torch.exp(g[:, t])                                   # [B,H,Dk] or [B,H]
        S = S * (a[:, :, None, :] if channel else a[:, :, None, None])
        kt, qt, vt = k[:, t], q[:, t], v[:, t]
        y = torch.einsum("bhij,bhj->bhi", S, kt)
        u = beta[:, t][..., None] * (vt - y)
        S = S + u[..., :, None] * kt[..., None, :]
        outs.append(scale * torch.einsum("bhij,bhj->bhi", S, qt))
    return torch.stack(outs, 1), S


def backward(q, k, v, g, beta, do, h0=None, dht=None, scale: float = 1.0):
    """Gradients (dq, dk, dv, dg, dbeta, dh0) as float64 numpy arrays for a
    fixed-length batch (layouts as ``forward``; do like v, dht like h0)."""
    import torch
    to = lambda x: torch.tensor(_f64(x), dtype=torch.float64, requires_grad=True)  # noqa: E731
    qt, kt, vt, gt, bt = (to(x) for x in (q, k, v, g, beta))
    B, T, H, Dk = qt.shape
    Dv = vt.shape[-1]
    h0t = to(h0) if h0 is not None else torch.zeros((B, H, Dv, Dk), dtype=torch.float64,
                                                     requires_grad=True)
    o, ST = forward_torch(qt, kt, vt, gt, bt, h0t, scale)
    loss = (o * torch.tensor(_f64(do))).sum()
    if dht is not None:
        loss = loss + (ST * torch.tensor(_f64(dht))).sum()
    grads = torch.autograd.grad(loss, [qt, kt, vt, gt, bt, h0t], allow_unused=True)
    return tuple(np.zeros(x.shape) if gr is None else gr.detach().numpy()
                 for gr, x in zip(grads, (qt, kt, vt, gt, bt, h0t)))
