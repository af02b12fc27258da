"""gated_delta_rule_44_amd -- the gated delta-rule hot path on MI355X.

A thin ctypes binding over libgdr.so (include/gdr.h).  It only checks torch
tensors, allocates outputs with torch, and passes raw device pointers and the
current HIP stream to the library; every step of the computation runs in the
library's HIP kernels.  There is no fallback: if libgdr.so is missing or was
built for another GPU, calls raise.

Recurrence (Kimi Delta Attention: per-key-channel gate; Gated DeltaNet: one
scalar gate per head -- "Super Apriel: One Checkpoint, Many Speeds",
gist.science summary section 2a), with the gate passed as g = ln a:
    S_t = S_{t-1} Diag(a_t)(I - beta_t k_t k_t^T) + beta_t v_t k_t^T
    o_t = scale * S_t q_t
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = ["prefill", "prefill_varlen", "prefill_varlen_pool", "decode_step",
           "decode_placement", "decode_tokens", "decode_commit", "workspace_bytes",
           "prefill_fused", "prefill_varlen_fused", "decode_tokens_fused",
           "fused_workspace_bytes", "backward", "backward_varlen", "version", "GdrError",
           "lib_path",
           "FA", "SWA", "GDN", "KDA"]

FA, SWA, GDN, KDA = 0, 1, 2, 3
_F32, _BF16 = 0, 1
_SCALAR, _CHANNEL = 0, 1
_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libgdr.so")
_lib = None


class GdrError(RuntimeError):
    """A libgdr call returned a non-OK status."""


def lib_path() -> str:
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise GdrError("libgdr.so is not built (%s); run "
                       "`python -m gated_delta_rule_44_amd.build`" % _LIB_PATH)
    lib = ctypes.CDLL(_LIB_PATH)
    P, I, F, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.gdr_last_error.restype = ctypes.c_char_p
    lib.gdr_version.restype = ctypes.c_char_p
    lib.gdr_prefill_workspace_bytes.restype = Z
    lib.gdr_prefill_workspace_bytes.argtypes = [I, I, I, ctypes.c_longlong, I]
    lib.gdr_prefill_chunked.restype = I
    lib.gdr_prefill_chunked.argtypes = [I, I, I, I, I, I, I, I, F,
                                        P, P, P, P, P, P, P, P, P, Z, P]
    lib.gdr_prefill_chunked_noalloc.restype = I
    lib.gdr_prefill_chunked_noalloc.argtypes = [I, I, I, I, I, I, I, I, F,
                                                P, P, P, P, P, P, P, P, P]
    lib.gdr_prefill_chunked_varlen.restype = I
    lib.gdr_prefill_chunked_varlen.argtypes = [I, I, I, I, I, I, I, I, F, P, P,
                                               P, P, P, P, P, P, P, P, P, Z, P]
    lib.gdr_decode_step.restype = I
    lib.gdr_decode_step.argtypes = [I, I, I, I, I, I, F, P, P, P, P, P, P, P, P]
    lib.gdr_decode_placement.restype = I
    lib.gdr_decode_placement.argtypes = [P, I, I, I, I, I, I, F,
                                         P, P, P, P, P, P, P, P]
    lib.gdr_prefill_varlen_pool.restype = I
    lib.gdr_prefill_varlen_pool.argtypes = [I, I, I, I, I, I, I, I, F, P, P,
                                            P, P, P, P, P, I, P, P, P, P, P, P,
                                            P, Z, P]
    lib.gdr_decode_tokens.restype = I
    lib.gdr_decode_tokens.argtypes = [I, I, I, I, I, I, I, F, P, P, P, P, P,
                                      P, P, I, P, P, P, P]
    lib.gdr_decode_commit.restype = I
    lib.gdr_decode_commit.argtypes = [I, I, I, I, I, P, I, P, P, P, P]
    lib.gdr_prefill_fused_workspace_bytes.restype = Z
    lib.gdr_prefill_fused_workspace_bytes.argtypes = [I, I, I, ctypes.c_longlong, I]
    lib.gdr_prefill_chunked_fused.restype = I
    lib.gdr_prefill_chunked_fused.argtypes = [I, I, I, I, I, I, I, I, F,
                                              P, P, P, P, P, F, P, P, P, P, Z, P]
    lib.gdr_prefill_varlen_fused.restype = I
    lib.gdr_prefill_varlen_fused.argtypes = [I, I, I, I, I, I, I, I, F, P, P,
                                             P, P, P, P, P, F, P, P, P, P, Z, P]
    lib.gdr_backward_workspace_bytes.restype = Z
    lib.gdr_backward_workspace_bytes.argtypes = [I, I, I, I, I, I]
    lib.gdr_backward_chunked.restype = I
    lib.gdr_backward_chunked.argtypes = [I, I, I, I, I, I, I, I, F, P, P, P, P, P, P, P, P,
                                         P, P, P, P, P, P, P, Z, P]
    lib.gdr_decode_tokens_fused.restype = I
    lib.gdr_decode_tokens_fused.argtypes = [I, I, I, I, I, I, I, F, P, P, P, P, P, F,
                                            P, P, I, P, P, P, P]
    lib.gdr_backward_varlen_workspace_bytes.restype = Z
    lib.gdr_backward_varlen_workspace_bytes.argtypes = [I, I, ctypes.c_longlong, I, I, I]
    lib.gdr_backward_chunked_varlen.restype = I
    lib.gdr_backward_chunked_varlen.argtypes = [I, I, I, I, I, I, I, I, F, P, P, P, P, P, P,
                                                P, P, P, P, P, P, P, P, P, P, P, Z, P]
    _lib = lib
    return lib


def version() -> str:
    return _load().gdr_version().decode()


def workspace_bytes(dtype, gated_channels: bool, n_seqs: int, tokens: int,
                    heads: int) -> int:
    """Bytes of device workspace a prefill over n_seqs sequences of `tokens`
    tokens in all needs (include/gdr.h, gdr_prefill_workspace_bytes)."""
    dt = _BF16 if dtype == torch.bfloat16 else _F32
    gk = _CHANNEL if gated_channels else _SCALAR
    return int(_load().gdr_prefill_workspace_bytes(dt, gk, int(n_seqs), int(tokens),
                                                   int(heads)))


def _workspace(workspace, nbytes, dev):
    if workspace is None:
        return torch.empty(max(nbytes, 1), device=dev, dtype=torch.uint8)
    _dense("workspace", workspace, device=dev)
    _need(workspace.numel() * workspace.element_size() >= nbytes,
          "workspace too small: %d bytes needed" % nbytes)
    return workspace


def _check(rc: int):
    if rc != 0:
        raise GdrError("libgdr status %d: %s" % (rc, _load().gdr_last_error().decode()))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return _BF16
    if t.dtype == torch.float32:
        return _F32
    raise GdrError("q/k/v must be bfloat16 or float32, got %s" % t.dtype)


def _need(cond, msg):
    if not cond:
        raise GdrError(msg)


def _dense(name, t, dtype=None, device=None):
    _need(isinstance(t, torch.Tensor), "%s must be a torch.Tensor" % name)
    _need(t.is_cuda, "%s must be a GPU tensor" % name)
    _need(t.is_contiguous(), "%s must be contiguous" % name)
    if dtype is not None:
        _need(t.dtype == dtype, "%s must be %s, got %s" % (name, dtype, t.dtype))
    if device is not None:
        _need(t.device == device, "%s is on %s, expected %s" % (name, t.device, device))


def prefill(q, k, v, g, beta, h0=None, scale: float = 1.0,
            output_final_state: bool = True, ht=None, workspace=None):
    """Chunked prefill, fixed-length batch.

    q, k [B,T,H,D], v [B,T,H,D] (bf16: chunked MFMA path; fp32: recurrent
    path), g [B,T,H] (scalar gate) or [B,T,H,D] (channel gate) fp32 log
    gates, beta [B,T,H] fp32, h0 [B,H,D,D] fp32 or None.
    Returns (o [B,T,H,D], ht [B,H,D,D] fp32 or None).  ``ht`` may be passed
    in (it may be h0 itself for an in-place resume); ``workspace`` (a device
    buffer of workspace_bytes(...) bytes) is allocated when not given.
    """
    B, T, H, D = q.shape
    dev = q.device
    for n, t in (("q", q), ("k", k), ("v", v)):
        _dense(n, t, q.dtype, dev)
    _dense("g", g, torch.float32, dev)
    _dense("beta", beta, torch.float32, dev)
    _need(k.shape == q.shape and v.shape == q.shape, "q, k, v shapes differ")
    _need(beta.shape == (B, T, H), "beta must be [B,T,H]")
    if g.dim() == 4:
        _need(g.shape == (B, T, H, D), "channel gate must be [B,T,H,D]")
        gk = _CHANNEL
    else:
        _need(g.shape == (B, T, H), "scalar gate must be [B,T,H]")
        gk = _SCALAR
    if h0 is not None:
        _dense("h0", h0, torch.float32, dev)
        _need(h0.shape == (B, H, D, D), "h0 must be [B,H,D,D]")
    o = torch.empty_like(v)
    if output_final_state and ht is None:
        ht = torch.empty((B, H, D, D), device=dev, dtype=torch.float32)
    if ht is not None:
        _dense("ht", ht, torch.float32, dev)
        _need(ht.shape == (B, H, D, D), "ht must be [B,H,D,D]")
    nbytes = workspace_bytes(q.dtype, gk == _CHANNEL, B, B * T, H)
    workspace = _workspace(workspace, nbytes, dev)
    _check(_load().gdr_prefill_chunked(
        _dt(q), gk, B, T, H, D, D, 64, float(scale), _ptr(q), _ptr(k), _ptr(v),
        _ptr(g), _ptr(beta), _ptr(h0), _ptr(o), _ptr(ht), _ptr(workspace), nbytes,
        _stream(dev)))
    return o, ht


# the library's own per-GPU workspace for prefill_noalloc (include/gdr.h,
# GDR_NOALLOC_MAX_BYTES)
NOALLOC_MAX_BYTES = 32 << 20


def prefill_noalloc(q, k, v, g, beta, o, h0=None, ht=None, scale: float = 1.0):
    """prefill() through gdr_prefill_chunked_noalloc, which takes no
    workspace (the library keeps one array of NOALLOC_MAX_BYTES per GPU) and
    allocates nothing; o [B,T,H,D] and ht [B,H,D,D] fp32 (or None) are the
    caller's, so this call allocates nothing either.  Calls that overlap on
    one GPU race on that array."""
    B, T, H, D = q.shape
    dev = q.device
    for n, t in (("q", q), ("k", k), ("v", v), ("o", o)):
        _dense(n, t, q.dtype, dev)
    _dense("g", g, torch.float32, dev)
    _dense("beta", beta, torch.float32, dev)
    _need(k.shape == q.shape and v.shape == q.shape and o.shape == q.shape,
          "q, k, v, o shapes differ")
    _need(beta.shape == (B, T, H), "beta must be [B,T,H]")
    if g.dim() == 4:
        _need(g.shape == (B, T, H, D), "channel gate must be [B,T,H,D]")
        gk = _CHANNEL
    else:
        _need(g.shape == (B, T, H), "scalar gate must be [B,T,H]")
        gk = _SCALAR
    for n, t in (("h0", h0), ("ht", ht)):
        if t is not None:
            _dense(n, t, torch.float32, dev)
            _need(t.shape == (B, H, D, D), "%s must be [B,H,D,D]" % n)
    _check(_load().gdr_prefill_chunked_noalloc(
        _dt(q), gk, B, T, H, D, D, 64, float(scale), _ptr(q), _ptr(k), _ptr(v),
        _ptr(g), _ptr(beta), _ptr(h0), _ptr(o), _ptr(ht), _stream(dev)))
    return o, ht


def prefill_varlen(q, k, v, g, beta, cu_seqlens, h0=None, scale: float = 1.0,
                   cu_seqlens_host=None, output_final_state: bool = True,
                   workspace=None, ht=None):
    """Chunked prefill over a packed batch.

    q, k, v [T_tot,H,D], g [T_tot,H] or [T_tot,H,D], beta [T_tot,H],
    cu_seqlens int32 [N+1] on the GPU, h0 [N,H,D,D] or None.  When
    cu_seqlens_host (a host int32 sequence) is given the library validates
    it.  Returns (o [T_tot,H,D], ht [N,H,D,D] or None).
    """
    Tt, H, D = q.shape
    dev = q.device
    for n, t in (("q", q), ("k", k), ("v", v)):
        _dense(n, t, q.dtype, dev)
    _dense("g", g, torch.float32, dev)
    _dense("beta", beta, torch.float32, dev)
    _dense("cu_seqlens", cu_seqlens, torch.int32, dev)
    N = cu_seqlens.numel() - 1
    gk = _CHANNEL if g.dim() == 3 else _SCALAR
    _need(g.shape == ((Tt, H, D) if gk == _CHANNEL else (Tt, H)), "bad gate shape")
    _need(beta.shape == (Tt, H), "beta must be [T_tot,H]")
    if h0 is not None:
        _dense("h0", h0, torch.float32, dev)
        _need(h0.shape == (N, H, D, D), "h0 must be [N,H,D,D]")
    host = None
    if cu_seqlens_host is not None:
        import numpy as np
        host = np.ascontiguousarray(np.asarray(cu_seqlens_host, dtype=np.int32))
        _need(host.shape == (N + 1,), "cu_seqlens_host must have N+1 entries")
    o = torch.empty_like(v)
    if output_final_state and ht is None:
        ht = torch.empty((N, H, D, D), device=dev, dtype=torch.float32)
    nbytes = workspace_bytes(q.dtype, gk == _CHANNEL, N, Tt, H)
    workspace = _workspace(workspace, nbytes, dev)
    hp = None if host is None else host.ctypes.data_as(ctypes.c_void_p)
    _check(_load().gdr_prefill_chunked_varlen(
        _dt(q), gk, N, Tt, H, D, D, 64, float(scale), _ptr(cu_seqlens), hp,
        _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(h0), _ptr(o),
        _ptr(ht), _ptr(workspace), nbytes, _stream(dev)))
    return o, ht


def decode_step(q, k, v, g, beta, state, scale: float = 1.0, o=None):
    """One token: q, k, v [B,H,D], g [B,H] or [B,H,D], beta [B,H], state
    [B,H,D,D] fp32 updated in place.  Returns o [B,H,D]."""
    B, H, D = q.shape
    dev = q.device
    for n, t in (("q", q), ("k", k), ("v", v)):
        _dense(n, t, q.dtype, dev)
    _dense("g", g, torch.float32, dev)
    _dense("beta", beta, torch.float32, dev)
    _dense("state", state, torch.float32, dev)
    _need(state.shape == (B, H, D, D), "state must be [B,H,D,D]")
    gk = _CHANNEL if g.dim() == 3 else _SCALAR
    if o is None:
        o = torch.empty_like(v)
    _check(_load().gdr_decode_step(
        _dt(q), gk, B, H, D, D, float(scale), _ptr(q), _ptr(k), _ptr(v), _ptr(g),
        _ptr(beta), _ptr(state), _ptr(o), _stream(dev)))
    return o


def decode_placement(placement, q, k, v, g, beta, state_pool, scale: float = 1.0,
                     o=None):
    """One token through L layers: placement (host, L codes 0..3); q, k, v, g
    [L,B,H,D]; beta [L,B,H]; state_pool [L,B,H,D,D] updated in place for the
    layers tagged GDN (2) or KDA (3).  Returns o [L,B,H,D]; slots of other
    layers are left as they were (uninitialised if o is None)."""
    import numpy as np
    L, B, H, D = q.shape
    dev = q.device
    for n, t in (("q", q), ("k", k), ("v", v)):
        _dense(n, t, q.dtype, dev)
    _dense("g", g, torch.float32, dev)
    _dense("beta", beta, torch.float32, dev)
    _dense("state_pool", state_pool, torch.float32, dev)
    _need(g.shape == (L, B, H, D), "g must be [L,B,H,D]")
    _need(state_pool.shape == (L, B, H, D, D), "state_pool must be [L,B,H,D,D]")
    p = np.ascontiguousarray(np.asarray(placement, dtype=np.uint8))
    _need(p.shape == (L,), "placement must have L entries")
    if o is None:
        o = torch.empty_like(v)
    _check(_load().gdr_decode_placement(
        p.ctypes.data_as(ctypes.c_void_p), L, _dt(q), B, H, D, D, float(scale),
        _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(state_pool),
        _ptr(o), _stream(dev)))
    return o


def _host_i32(x, n, name):
    import numpy as np
    a = np.ascontiguousarray(np.asarray(x, dtype=np.int32))
    _need(a.shape == (n,), "%s must have %d entries" % (name, n))
    return a


def prefill_varlen_pool(q, k, v, g, beta, cu_seqlens, state_pool, h0_slot, ht_slot,
                        scale: float = 1.0, cu_seqlens_host=None, slots_host=None,
                        workspace=None):
    """Packed-batch prefill with states in a slot-indexed pool.

    As prefill_varlen, but sequence n starts from state_pool[h0_slot[n]]
    (zeros for slot -1) and its final state is written to
    state_pool[ht_slot[n]] (not stored for -1).  state_pool [P,H,D,D] fp32;
    h0_slot, ht_slot int32 [N] on the GPU.  slots_host = (h0 slots, ht slots)
    as host sequences makes the library validate them.  Returns o.
    """
    Tt, H, D = q.shape
    dev = q.device
    for n, t in (("q", q), ("k", k), ("v", v)):
        _dense(n, t, q.dtype, dev)
    _dense("g", g, torch.float32, dev)
    _dense("beta", beta, torch.float32, dev)
    _dense("cu_seqlens", cu_seqlens, torch.int32, dev)
    _dense("state_pool", state_pool, torch.float32, dev)
    N = cu_seqlens.numel() - 1
    _dense("h0_slot", h0_slot, torch.int32, dev)
    _dense("ht_slot", ht_slot, torch.int32, dev)
    _need(h0_slot.shape == (N,) and ht_slot.shape == (N,), "slot maps must be [N]")
    gk = _CHANNEL if g.dim() == 3 else _SCALAR
    _need(g.shape == ((Tt, H, D) if gk == _CHANNEL else (Tt, H)), "bad gate shape")
    _need(beta.shape == (Tt, H), "beta must be [T_tot,H]")
    _need(state_pool.dim() == 4 and state_pool.shape[1:] == (H, D, D),
          "state_pool must be [P,H,D,D]")
    host = None if cu_seqlens_host is None else _host_i32(cu_seqlens_host, N + 1,
                                                           "cu_seqlens_host")
    h0h = hth = None
    if slots_host is not None:
        h0h = _host_i32(slots_host[0], N, "h0 slots")
        hth = _host_i32(slots_host[1], N, "ht slots")
    o = torch.empty_like(v)
    nbytes = workspace_bytes(q.dtype, gk == _CHANNEL, N, Tt, H)
    workspace = _workspace(workspace, nbytes, dev)
    hp = lambda a: None if a is None else a.ctypes.data_as(ctypes.c_void_p)  # noqa: E731
    _check(_load().gdr_prefill_varlen_pool(
        _dt(q), gk, N, Tt, H, D, D, 64, float(scale), _ptr(cu_seqlens), hp(host),
        _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), state_pool.shape[0],
        _ptr(state_pool), _ptr(h0_slot), _ptr(ht_slot), hp(h0h), hp(hth), _ptr(o),
        _ptr(workspace), nbytes, _stream(dev)))
    return o


def decode_tokens(q, k, v, g, beta, state_pool, slot=None, checkpoints=None,
                  scale: float = 1.0, slot_host=None, o=None):
    """n tokens per sequence in one launch.

    q, k, v [B,n,H,D]; g [B,n,H] or [B,n,H,D]; beta [B,n,H]; state_pool
    [P,H,D,D] fp32; slot int32 [B] on the GPU (None: slot b; -1: idle).
    checkpoints: None (the pool is advanced in place), True (allocate) or a
    [B,n,H,D,D] fp32 tensor that receives the state after every token while
    the pool keeps its bytes.  Returns o, or (o, checkpoints) when
    checkpoints is given.
    """
    B, n, H, D = q.shape
    dev = q.device
    for nm, t in (("q", q), ("k", k), ("v", v)):
        _dense(nm, t, q.dtype, dev)
    _dense("g", g, torch.float32, dev)
    _dense("beta", beta, torch.float32, dev)
    _dense("state_pool", state_pool, torch.float32, dev)
    _need(k.shape == q.shape and v.shape == q.shape, "q, k, v shapes differ")
    _need(beta.shape == (B, n, H), "beta must be [B,n,H]")
    gk = _CHANNEL if g.dim() == 4 else _SCALAR
    _need(g.shape == ((B, n, H, D) if gk == _CHANNEL else (B, n, H)), "bad gate shape")
    _need(state_pool.dim() == 4 and state_pool.shape[1:] == (H, D, D),
          "state_pool must be [P,H,D,D]")
    if slot is not None:
        _dense("slot", slot, torch.int32, dev)
        _need(slot.shape == (B,), "slot must be [B]")
    sh = None if slot_host is None else _host_i32(slot_host, B, "slot_host")
    ret_ckpt = checkpoints is not None
    if checkpoints is True:
        checkpoints = torch.empty((B, n, H, D, D), device=dev, dtype=torch.float32)
    if ret_ckpt:
        _dense("checkpoints", checkpoints, torch.float32, dev)
        _need(checkpoints.shape == (B, n, H, D, D), "checkpoints must be [B,n,H,D,D]")
    if o is None:
        o = torch.empty_like(v)
    _check(_load().gdr_decode_tokens(
        _dt(q), gk, B, n, H, D, D, float(scale), _ptr(q), _ptr(k), _ptr(v), _ptr(g),
        _ptr(beta), _ptr(slot), None if sh is None else sh.ctypes.data_as(ctypes.c_void_p),
        state_pool.shape[0], _ptr(state_pool), _ptr(checkpoints if ret_ckpt else None),
        _ptr(o), _stream(dev)))
    return (o, checkpoints) if ret_ckpt else o


def decode_commit(checkpoints, accepted, state_pool, slot=None):
    """Keep the state after the accepted prefix: for 1 <= accepted[b] <= n the
    pool slot of sequence b receives checkpoints[b, accepted[b]-1]; other
    counts leave it.  checkpoints [B,n,H,D,D], accepted int32 [B] on the GPU."""
    B, n, H, D, _ = checkpoints.shape
    dev = checkpoints.device
    _dense("checkpoints", checkpoints, torch.float32, dev)
    _dense("accepted", accepted, torch.int32, dev)
    _dense("state_pool", state_pool, torch.float32, dev)
    _need(accepted.shape == (B,), "accepted must be [B]")
    _need(state_pool.dim() == 4 and state_pool.shape[1:] == (H, D, D),
          "state_pool must be [P,H,D,D]")
    if slot is not None:
        _dense("slot", slot, torch.int32, dev)
        _need(slot.shape == (B,), "slot must be [B]")
    _check(_load().gdr_decode_commit(
        B, n, H, D, D, _ptr(slot), state_pool.shape[0], _ptr(accepted),
        _ptr(checkpoints), _ptr(state_pool), _stream(dev)))


# --------------------------------------------------------------------------
# Fused input preprocessing: raw projections in, the kernels normalise q and
# k per token and form beta = sigmoid(beta_logit) and
# g = -gate_scale * softplus(gate_logit).  Logits share the dtype of q.

def fused_workspace_bytes(dtype, gated_channels: bool, n_seqs: int, tokens: int,
                          heads: int) -> int:
    return int(_load().gdr_prefill_fused_workspace_bytes(
        _BF16 if dtype == torch.bfloat16 else _F32, _CHANNEL if gated_channels else _SCALAR,
        n_seqs, tokens, heads))


def _raw_checks(q, k, v, gate_logit, beta_logit, lead):
    dev = q.device
    for n, t in (("q", q), ("k", k), ("v", v), ("gate_logit", gate_logit),
                 ("beta_logit", beta_logit)):
        _dense(n, t, q.dtype, dev)
    D = q.shape[-1]
    _need(k.shape == q.shape and v.shape == q.shape, "q, k, v shapes differ")
    _need(tuple(beta_logit.shape) == lead, "beta_logit must be %s" % (lead,))
    if tuple(gate_logit.shape) == lead + (D,):
        return _CHANNEL
    _need(tuple(gate_logit.shape) == lead, "gate_logit must be %s or %s" % (lead, lead + (D,)))
    return _SCALAR


def prefill_fused(q, k, v, gate_logit, beta_logit, gate_scale: float, h0=None,
                  scale: float = 1.0, output_final_state: bool = True, ht=None,
                  workspace=None):
    """prefill() on raw projections: q, k, v [B,T,H,D]; gate_logit [B,T,H] or
    [B,T,H,D] and beta_logit [B,T,H] in the dtype of q.  Returns (o, ht)."""
    B, T, H, D = q.shape
    dev = q.device
    gk = _raw_checks(q, k, v, gate_logit, beta_logit, (B, T, H))
    if h0 is not None:
        _dense("h0", h0, torch.float32, dev)
        _need(h0.shape == (B, H, D, D), "h0 must be [B,H,D,D]")
    o = torch.empty_like(v)
    if output_final_state and ht is None:
        ht = torch.empty((B, H, D, D), device=dev, dtype=torch.float32)
    if ht is not None:
        _dense("ht", ht, torch.float32, dev)
        _need(ht.shape == (B, H, D, D), "ht must be [B,H,D,D]")
    nbytes = fused_workspace_bytes(q.dtype, gk == _CHANNEL, B, B * T, H)
    workspace = _workspace(workspace, nbytes, dev)
    _check(_load().gdr_prefill_chunked_fused(
        _dt(q), gk, B, T, H, D, D, 64, float(scale), _ptr(q), _ptr(k), _ptr(v),
        _ptr(gate_logit), _ptr(beta_logit), float(gate_scale), _ptr(h0), _ptr(o), _ptr(ht),
        _ptr(workspace), nbytes, _stream(dev)))
    return o, ht


def prefill_varlen_fused(q, k, v, gate_logit, beta_logit, gate_scale: float, cu_seqlens,
                         h0=None, scale: float = 1.0, cu_seqlens_host=None,
                         output_final_state: bool = True, workspace=None, ht=None):
    """prefill_varlen() on raw projections: q, k, v [T_tot,H,D]; gate_logit
    [T_tot,H] or [T_tot,H,D] and beta_logit [T_tot,H] in the dtype of q."""
    Tt, H, D = q.shape
    dev = q.device
    gk = _raw_checks(q, k, v, gate_logit, beta_logit, (Tt, H))
    _dense("cu_seqlens", cu_seqlens, torch.int32, dev)
    N = cu_seqlens.numel() - 1
    if h0 is not None:
        _dense("h0", h0, torch.float32, dev)
        _need(h0.shape == (N, H, D, D), "h0 must be [N,H,D,D]")
    host = None if cu_seqlens_host is None else _host_i32(cu_seqlens_host, N + 1,
                                                           "cu_seqlens_host")
    o = torch.empty_like(v)
    if output_final_state and ht is None:
        ht = torch.empty((N, H, D, D), device=dev, dtype=torch.float32)
    nbytes = fused_workspace_bytes(q.dtype, gk == _CHANNEL, N, Tt, H)
    workspace = _workspace(workspace, nbytes, dev)
    _check(_load().gdr_prefill_varlen_fused(
        _dt(q), gk, N, Tt, H, D, D, 64, float(scale), _ptr(cu_seqlens),
        None if host is None else host.ctypes.data_as(ctypes.c_void_p),
        _ptr(q), _ptr(k), _ptr(v), _ptr(gate_logit), _ptr(beta_logit), float(gate_scale),
        _ptr(h0), _ptr(o), _ptr(ht), _ptr(workspace), nbytes, _stream(dev)))
    return o, ht


def decode_tokens_fused(q, k, v, gate_logit, beta_logit, gate_scale: float, state_pool,
                        slot=None, checkpoints=None, scale: float = 1.0, slot_host=None,
                        o=None):
    """decode_tokens() on raw projections: q, k, v [B,n,H,D]; gate_logit
    [B,n,H] or [B,n,H,D] and beta_logit [B,n,H] in the dtype of q."""
    B, n, H, D = q.shape
    dev = q.device
    gk = _raw_checks(q, k, v, gate_logit, beta_logit, (B, n, H))
    _dense("state_pool", state_pool, torch.float32, dev)
    _need(state_pool.dim() == 4 and state_pool.shape[1:] == (H, D, D),
          "state_pool must be [P,H,D,D]")
    if slot is not None:
        _dense("slot", slot, torch.int32, dev)
        _need(slot.shape == (B,), "slot must be [B]")
    sh = None if slot_host is None else _host_i32(slot_host, B, "slot_host")
    ret_ckpt = checkpoints is not None
    if checkpoints is True:
        checkpoints = torch.empty((B, n, H, D, D), device=dev, dtype=torch.float32)
    if ret_ckpt:
        _dense("checkpoints", checkpoints, torch.float32, dev)
        _need(checkpoints.shape == (B, n, H, D, D), "checkpoints must be [B,n,H,D,D]")
    if o is None:
        o = torch.empty_like(v)
    _check(_load().gdr_decode_tokens_fused(
        _dt(q), gk, B, n, H, D, D, float(scale), _ptr(q), _ptr(k), _ptr(v),
        _ptr(gate_logit), _ptr(beta_logit), float(gate_scale), _ptr(slot),
        None if sh is None else sh.ctypes.data_as(ctypes.c_void_p), state_pool.shape[0],
        _ptr(state_pool), _ptr(checkpoints if ret_ckpt else None), _ptr(o), _stream(dev)))
    return (o, checkpoints) if ret_ckpt else o


def backward(q, k, v, g, beta, do, h0=None, dht=None, scale: float = 1.0,
             workspace=None):
    """Gradients of prefill() for a fixed-length bf16 batch.

    q, k, v, do [B,T,H,D] bf16; g [B,T,H] or [B,T,H,D] and beta [B,T,H]
    fp32; h0 and dht [B,H,D,D] fp32 or None.  Returns fp32
    (dq, dk, dv, dg, dbeta, dh0)."""
    B, T, H, D = q.shape
    dev = q.device
    for n, t in (("q", q), ("k", k), ("v", v), ("do", do)):
        _dense(n, t, torch.bfloat16, dev)
    _dense("g", g, torch.float32, dev)
    _dense("beta", beta, torch.float32, dev)
    _need(k.shape == q.shape and v.shape == q.shape and do.shape == q.shape, "shapes differ")
    _need(beta.shape == (B, T, H), "beta must be [B,T,H]")
    gk = _CHANNEL if g.dim() == 4 else _SCALAR
    _need(g.shape == ((B, T, H, D) if gk == _CHANNEL else (B, T, H)), "bad gate shape")
    for n, t in (("h0", h0), ("dht", dht)):
        if t is not None:
            _dense(n, t, torch.float32, dev)
            _need(t.shape == (B, H, D, D), "%s must be [B,H,D,D]" % n)
    f32 = dict(device=dev, dtype=torch.float32)
    dq, dk, dv = (torch.empty((B, T, H, D), **f32) for _ in range(3))
    dg = torch.empty(g.shape, **f32)
    dbeta = torch.empty((B, T, H), **f32)
    dh0 = torch.empty((B, H, D, D), **f32)
    nbytes = int(_load().gdr_backward_workspace_bytes(gk, B, T, H, D, D))
    workspace = _workspace(workspace, nbytes, dev)
    _check(_load().gdr_backward_chunked(
        _BF16, gk, B, T, H, D, D, 64, float(scale), _ptr(q), _ptr(k), _ptr(v), _ptr(g),
        _ptr(beta), _ptr(h0), _ptr(do), _ptr(dht), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dg),
        _ptr(dbeta), _ptr(dh0), _ptr(workspace), nbytes, _stream(dev)))
    return dq, dk, dv, dg, dbeta, dh0


def backward_varlen(q, k, v, g, beta, do, cu_seqlens, h0=None, dht=None, scale: float = 1.0,
                    cu_seqlens_host=None, workspace=None):
    """Gradients of prefill_varlen() for a packed bf16 batch.

    q, k, v, do [T_tot,H,D] bf16; g [T_tot,H] or [T_tot,H,D] and beta
    [T_tot,H] fp32; cu_seqlens int32 [N+1] on the GPU; h0 and dht [N,H,D,D]
    fp32 or None.  Returns fp32 (dq, dk, dv, dg, dbeta, dh0)."""
    Tt, H, D = q.shape
    dev = q.device
    for n, t in (("q", q), ("k", k), ("v", v), ("do", do)):
        _dense(n, t, torch.bfloat16, dev)
    _dense("g", g, torch.float32, dev)
    _dense("beta", beta, torch.float32, dev)
    _dense("cu_seqlens", cu_seqlens, torch.int32, dev)
    N = cu_seqlens.numel() - 1
    _need(k.shape == q.shape and v.shape == q.shape and do.shape == q.shape, "shapes differ")
    _need(beta.shape == (Tt, H), "beta must be [T_tot,H]")
    gk = _CHANNEL if g.dim() == 3 else _SCALAR
    _need(g.shape == ((Tt, H, D) if gk == _CHANNEL else (Tt, H)), "bad gate shape")
    for n, t in (("h0", h0), ("dht", dht)):
        if t is not None:
            _dense(n, t, torch.float32, dev)
            _need(t.shape == (N, H, D, D), "%s must be [N,H,D,D]" % n)
    host = None
    if cu_seqlens_host is not None:
        import numpy as np
        host = np.ascontiguousarray(np.asarray(cu_seqlens_host, dtype=np.int32))
        _need(host.shape == (N + 1,), "cu_seqlens_host must have N+1 entries")
    f32 = dict(device=dev, dtype=torch.float32)
    dq, dk, dv = (torch.empty((Tt, H, D), **f32) for _ in range(3))
    dg = torch.empty(g.shape, **f32)
    dbeta = torch.empty((Tt, H), **f32)
    dh0 = torch.empty((N, H, D, D), **f32)
    nbytes = int(_load().gdr_backward_varlen_workspace_bytes(gk, N, Tt, H, D, D))
    workspace = _workspace(workspace, nbytes, dev)
    hp = None if host is None else host.ctypes.data_as(ctypes.c_void_p)
    _check(_load().gdr_backward_chunked_varlen(
        _BF16, gk, N, Tt, H, D, D, 64, float(scale), _ptr(cu_seqlens), hp, _ptr(q), _ptr(k),
        _ptr(v), _ptr(g), _ptr(beta), _ptr(h0), _ptr(do), _ptr(dht), _ptr(dq), _ptr(dk),
        _ptr(dv), _ptr(dg), _ptr(dbeta), _ptr(dh0), _ptr(workspace), nbytes, _stream(dev)))
    return dq, dk, dv, dg, dbeta, dh0
