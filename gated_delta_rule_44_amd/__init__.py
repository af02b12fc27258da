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

__all__ = ["prefill", "prefill_varlen", "decode_step", "decode_placement",
           "workspace_bytes", "version", "GdrError", "lib_path",
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
    lib.gdr_prefill_chunked_varlen.restype = I
    lib.gdr_prefill_chunked_varlen.argtypes = [I, I, I, I, I, I, I, I, F, P, P,
                                               P, P, P, P, P, P, P, P, P, Z, P]
    lib.gdr_decode_step.restype = I
    lib.gdr_decode_step.argtypes = [I, I, I, I, I, I, F, P, P, P, P, P, P, P, P]
    lib.gdr_decode_placement.restype = I
    lib.gdr_decode_placement.argtypes = [P, I, I, I, I, I, I, F,
                                         P, P, P, P, P, P, P, P]
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
