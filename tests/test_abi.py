"""CPU tests of the C ABI: the library loads without a GPU, exports every
symbol include/gdr.h declares, and rejects bad arguments on the host before
any HIP call (no compute is launched here)."""
import ctypes
import os
import re

import numpy as np
import pytest
import torch

import gated_delta_rule_44_amd as gdr

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdr.h")
EINVAL, EUNSUPPORTED = 1, 2


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(gdr.lib_path()):
        pytest.skip("libgdr.so not built")
    return gdr._load()


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(gdr_[a-z_]+)\s*\(", src)))


def test_header_declares_the_boundary():
    names = declared_functions()
    assert names == sorted(["gdr_prefill_workspace_bytes", "gdr_prefill_chunked",
                            "gdr_prefill_chunked_noalloc",
                            "gdr_prefill_chunked_varlen", "gdr_decode_step",
                            "gdr_decode_placement", "gdr_prefill_varlen_pool",
                            "gdr_decode_tokens", "gdr_decode_commit",
                            "gdr_prefill_fused_workspace_bytes", "gdr_prefill_chunked_fused",
                            "gdr_prefill_varlen_fused", "gdr_decode_tokens_fused",
                            "gdr_backward_workspace_bytes", "gdr_backward_chunked",
                            "gdr_backward_varlen_workspace_bytes",
                            "gdr_backward_chunked_varlen",
                            "gdr_last_error", "gdr_version"])


def test_library_exports_every_declared_symbol(lib):
    raw = ctypes.CDLL(gdr.lib_path())
    for name in declared_functions():
        assert hasattr(raw, name), name


def test_version_and_workspace(lib):
    assert gdr.version().startswith("gdr")
    bf, f32 = torch.bfloat16, torch.float32
    # schedule and chunk offsets: N and N+1 int32, each rounded up to 256 bytes
    assert gdr.workspace_bytes(f32, False, 0, 0, 4) == 0
    assert gdr.workspace_bytes(f32, False, 1, 100, 4) == 512
    assert gdr.workspace_bytes(f32, True, 65, 100, 4) == 512 + 512
    # bf16, channel gate: + one int32 per (sequence, head), rounded up to 256
    # bytes (the pairs the plain pass leaves to the reference pass)
    assert gdr.workspace_bytes(bf, True, 64, 100, 4) == 256 + 512 + 1024
    assert gdr.workspace_bytes(bf, True, 2, 2 * 8192, 32) == 256 + 256 + 256
    assert gdr.workspace_bytes(f32, False, 2, 100, 0) == 0
    # bf16, scalar gate: + 5888 bytes (T and decay factors) per (chunk, head), for
    # tokens // 64 + N chunks
    assert gdr.workspace_bytes(bf, False, 1, 64, 1) == 512 + 2 * 5888
    assert gdr.workspace_bytes(bf, False, 4, 4 * 4096, 16) == 512 + (256 + 4) * 16 * 5888


F = ctypes.c_float
FAKE = 1 << 20          # aligned, never dereferenced: validation fails first
MIS = FAKE + 4          # misaligned


def prefill(lib, dt=1, gk=0, B=1, T=64, H=1, Dk=128, Dv=128, chunk=64, q=FAKE,
            k=FAKE, v=FAKE, g=FAKE, beta=FAKE, h0=None, o=FAKE, ht=FAKE, ws=FAKE,
            ws_bytes=1 << 30):
    return lib.gdr_prefill_chunked(dt, gk, B, T, H, Dk, Dv, chunk, F(1.0), q, k,
                                   v, g, beta, h0, o, ht, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,code,msg", [
    (dict(dt=7), EINVAL, "dtype"),
    (dict(gk=3), EINVAL, "gate kind"),
    (dict(Dk=128, Dv=64), EUNSUPPORTED, "Dk"),
    (dict(Dk=96, Dv=96), EUNSUPPORTED, "supported widths"),
    (dict(chunk=32), EUNSUPPORTED, "chunk"),
    (dict(B=-1), EINVAL, "bad sizes"),
    (dict(T=-5), EINVAL, "bad sizes"),
    (dict(H=0), EINVAL, "bad sizes"),
    (dict(B=1 << 20, T=1, H=1 << 9), EUNSUPPORTED, "(sequence, head) pairs exceed"),
    (dict(q=None), EINVAL, "q is NULL"),
    (dict(k=MIS), EINVAL, "k is not 16-byte aligned"),
    (dict(o=None), EINVAL, "o is NULL"),
    (dict(h0=MIS), EINVAL, "h0 is not 16-byte aligned"),
    (dict(h0=FAKE, ht=FAKE + 256), EINVAL, "overlap"),
    (dict(ws=None), EINVAL, "workspace of 12288 bytes needed, 0 given"),
    (dict(ws_bytes=12287), EINVAL, "workspace of 12288 bytes needed"),
    (dict(ws=MIS), EINVAL, "workspace is not 16-byte aligned"),
])
def test_prefill_rejects(lib, kw, code, msg):
    assert prefill(lib, **kw) == code
    assert msg in lib.gdr_last_error().decode()


def test_prefill_empty_batch_is_ok_without_gpu(lib):
    assert prefill(lib, B=0) == 0


def varlen(lib, N=2, Tt=10, cu=FAKE, host=None, ws=FAKE, ws_bytes=1 << 30, **kw):
    a = dict(dt=1, gk=1, H=1, Dk=128, Dv=128, chunk=64, q=FAKE, k=FAKE, v=FAKE,
             g=FAKE, beta=FAKE, h0=None, o=FAKE, ht=None)
    a.update(kw)
    hp = None if host is None else host.ctypes.data_as(ctypes.c_void_p)
    return lib.gdr_prefill_chunked_varlen(
        a["dt"], a["gk"], N, Tt, a["H"], a["Dk"], a["Dv"], a["chunk"], F(1.0),
        cu, hp, a["q"], a["k"], a["v"], a["g"], a["beta"], a["h0"], a["o"],
        a["ht"], ws, ws_bytes, None)


def test_varlen_rejects(lib):
    assert varlen(lib, cu=None) == EINVAL
    bad = np.array([0, 5, 3], np.int32)
    assert varlen(lib, Tt=3, host=bad) == EINVAL
    assert "decreases" in lib.gdr_last_error().decode()
    assert varlen(lib, Tt=9, host=np.array([0, 4, 10], np.int32)) == EINVAL
    assert "T_total" in lib.gdr_last_error().decode()
    assert varlen(lib, Tt=10, host=np.array([1, 4, 10], np.int32)) == EINVAL
    assert varlen(lib, ws=None) == EINVAL
    assert "workspace" in lib.gdr_last_error().decode()
    assert varlen(lib, ws_bytes=8) == EINVAL
    assert varlen(lib, N=0) == 0
    assert varlen(lib, N=1 << 20, H=1 << 9) == EUNSUPPORTED
    assert "pairs exceed" in lib.gdr_last_error().decode()


def test_decode_rejects(lib):
    args = lambda **kw: [kw.get("dt", 1), kw.get("gk", 1), kw.get("B", 2), 4,  # noqa: E731
                         kw.get("D", 128), kw.get("D", 128), F(1.0), FAKE, FAKE,
                         FAKE, FAKE, FAKE, kw.get("state", FAKE), FAKE, None]
    assert lib.gdr_decode_step(*args(D=32)) == EUNSUPPORTED
    assert lib.gdr_decode_step(*args(state=None)) == EINVAL
    assert lib.gdr_decode_step(*args(state=MIS)) == EINVAL
    assert lib.gdr_decode_step(*args(B=0)) == 0


def test_placement_rejects(lib):
    def call(p, L=None, **kw):
        p = np.asarray(p, np.uint8)
        L = len(p) if L is None else L
        return lib.gdr_decode_placement(
            p.ctypes.data_as(ctypes.c_void_p), L, 1, kw.get("B", 2), 4, 128, 128,
            F(1.0), FAKE, FAKE, FAKE, FAKE, FAKE, kw.get("pool", FAKE), FAKE, None)
    assert call([0, 1, 4]) == EINVAL
    assert "placement[2]" in lib.gdr_last_error().decode()
    assert call([0, 2], L=0) == EINVAL
    assert call([2, 3], pool=None) == EINVAL
    assert call([0, 1, 0]) == 0            # nothing recurrent: nothing to do
    assert lib.gdr_decode_placement(None, 3, 1, 2, 4, 128, 128, F(1.0), FAKE,
                                    FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == EINVAL


def _hp(a):
    return None if a is None else np.asarray(a, np.int32).ctypes.data_as(ctypes.c_void_p)


def tokens(lib, B=3, n=4, H=2, D=128, slot=FAKE, slot_host=None, pool=8, state=FAKE,
           ckpt=None, o=FAKE, q=FAKE):
    hs = None if slot_host is None else np.asarray(slot_host, np.int32)
    return lib.gdr_decode_tokens(1, 0, B, n, H, D, D, F(1.0), q, FAKE, FAKE, FAKE,
                                 FAKE, slot, None if hs is None else
                                 hs.ctypes.data_as(ctypes.c_void_p), pool, state,
                                 ckpt, o, None)


def test_decode_tokens_rejects(lib):
    err = lambda: lib.gdr_last_error().decode()  # noqa: E731
    assert tokens(lib, slot=None, pool=2) == EINVAL and "pool needs B = 3" in err()
    assert tokens(lib, slot_host=[0, 8, 1]) == EINVAL and "slot[1] = 8" in err()
    assert tokens(lib, slot_host=[0, -2, 1]) == EINVAL and "slot[1] = -2" in err()
    assert tokens(lib, slot_host=[5, 2, 5]) == EINVAL and "slot 5 is used by two" in err()
    assert tokens(lib, slot=None, slot_host=[0, 1, 2]) == EINVAL
    assert tokens(lib, state=None) == EINVAL and "state_pool is NULL" in err()
    assert tokens(lib, ckpt=MIS) == EINVAL
    assert tokens(lib, ckpt=FAKE + 4096) == EINVAL and "overlap" in err()
    assert tokens(lib, q=None) == EINVAL
    assert tokens(lib, D=96) == EUNSUPPORTED
    assert tokens(lib, B=-1) == EINVAL
    # nothing to do: no launch, no GPU needed
    assert tokens(lib, n=0) == 0
    assert tokens(lib, B=0, slot_host=[]) == 0


def test_decode_commit_rejects(lib):
    call = lambda **kw: lib.gdr_decode_commit(  # noqa: E731
        kw.get("B", 2), 3, 2, kw.get("D", 128), kw.get("D", 128), kw.get("slot", FAKE),
        kw.get("pool", 4), kw.get("acc", FAKE), kw.get("ckpt", FAKE),
        kw.get("state", FAKE), None)
    assert call(acc=None) == EINVAL and "accepted" in lib.gdr_last_error().decode()
    assert call(ckpt=None) == EINVAL
    assert call(state=MIS) == EINVAL
    assert call(slot=None, pool=1) == EINVAL
    assert call(D=32) == EUNSUPPORTED
    assert call(B=0) == 0


def pool_prefill(lib, N=2, h0s=FAKE, hts=FAKE, h0h=None, hth=None, pool=4, state=FAKE):
    return lib.gdr_prefill_varlen_pool(
        1, 1, N, 10, 1, 128, 128, 64, F(1.0), FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE,
        pool, state, h0s, hts, _hp(h0h), _hp(hth), FAKE, FAKE, 1 << 30, None)


def test_prefill_pool_rejects(lib):
    err = lambda: lib.gdr_last_error().decode()  # noqa: E731
    assert pool_prefill(lib, h0s=None) == EINVAL and "required" in err()
    assert pool_prefill(lib, state=None) == EINVAL
    assert pool_prefill(lib, h0h=[0, 4], hth=[1, 2]) == EINVAL and "h0_slot[1] = 4" in err()
    assert pool_prefill(lib, h0h=[0, 1], hth=[-3, 2]) == EINVAL and "ht_slot[0]" in err()
    assert pool_prefill(lib, h0h=[0, 1], hth=[3, 3]) == EINVAL and "both write slot 3" in err()
    assert pool_prefill(lib, h0h=[0, 1], hth=[1, 2]) == EINVAL and "reads slot 1" in err()
    assert pool_prefill(lib, pool=-1) == EINVAL
    assert pool_prefill(lib, N=0) == 0


def test_fused_rejects(lib):
    err = lambda: lib.gdr_last_error().decode()  # noqa: E731
    bf, f32 = torch.bfloat16, torch.float32
    # the fused records are 6144 bytes (two more factor rows)
    assert gdr.fused_workspace_bytes(bf, False, 1, 64, 1) == 512 + 2 * 6144
    assert gdr.fused_workspace_bytes(bf, True, 1, 64, 1) == gdr.workspace_bytes(bf, True, 1, 64, 1)
    assert gdr.fused_workspace_bytes(f32, False, 1, 64, 1) == 512

    def fixed(c=1.0, ws_bytes=1 << 30, **kw):
        return lib.gdr_prefill_chunked_fused(
            1, kw.get("gk", 0), 1, 64, 1, 128, 128, 64, F(1.0), FAKE, FAKE, FAKE,
            kw.get("xg", FAKE), kw.get("xb", FAKE), F(c), None, FAKE, FAKE, FAKE, ws_bytes, None)
    assert fixed(c=-0.5) == EINVAL and "gate_scale" in err()
    assert fixed(c=float("nan")) == EINVAL
    assert fixed(xg=None) == EINVAL and "g is NULL" in err()
    assert fixed(ws_bytes=512 + 2 * 6144 - 1) == EINVAL and "workspace of 12800" in err()

    def varlen_f(c=1.0, N=2, **kw):
        return lib.gdr_prefill_varlen_fused(
            1, 1, N, 10, 1, 128, 128, 64, F(1.0), FAKE, None, FAKE, FAKE, FAKE, FAKE, FAKE,
            F(c), None, FAKE, None, FAKE, 1 << 30, None)
    assert varlen_f(c=-1.0) == EINVAL
    assert varlen_f(N=0) == 0

    def tok(c=1.0, **kw):
        return lib.gdr_decode_tokens_fused(1, 1, 2, 3, 2, 128, 128, F(1.0), FAKE, FAKE, FAKE,
                                           FAKE, FAKE, F(c), None, None, kw.get("pool", 2),
                                           kw.get("state", FAKE), None, FAKE, None)
    assert tok(c=-2.0) == EINVAL
    assert tok(pool=1) == EINVAL and "pool needs" in err()
    assert tok(state=None) == EINVAL


def test_backward_rejects(lib):
    err = lambda: lib.gdr_last_error().decode()  # noqa: E731
    # chunk states and state gradients, the forward's workspace (for the
    # scalar gate: 5888-byte records; the forward stores no outputs) and per
    # (b, h, chunk) a record of Qt, Kb, W (bf16 64 x 128), P (bf16 64 x 64)
    # and e^{b_C} (fp32 128)
    st = 2 * 3 * 2 * 128 * 128 * 4
    rec = 2 * 3 * 2 * (3 * 64 * 128 * 2 + 64 * 64 * 2 + 128 * 4)
    # the forward's workspace: schedule, chunk offsets, one int32 per (sequence, head)
    # (rounded to 256 bytes), the records
    fwd_gdn = (512 + 256 + (200 // 64 + 2) * 3 * 5888 + 255) // 256 * 256
    # channel gate: the forward's workspace holds one int32 per (sequence, head) more
    assert lib.gdr_backward_workspace_bytes(1, 2, 100, 3, 128, 128) == 2 * st + 512 + 256 + rec
    assert lib.gdr_backward_workspace_bytes(0, 2, 100, 3, 128, 128) == 2 * st + fwd_gdn + rec
    assert lib.gdr_backward_workspace_bytes(1, 2, 0, 3, 128, 128) == 0

    def call(dt=1, ws_bytes=1 << 30, T=100, **kw):
        return lib.gdr_backward_chunked(
            dt, 1, 2, T, 3, 128, 128, 64, F(1.0), FAKE, FAKE, FAKE, FAKE, FAKE, None,
            kw.get("do", FAKE), None, FAKE, FAKE, FAKE, kw.get("dg", FAKE), FAKE, None,
            kw.get("ws", FAKE), ws_bytes, None)
    assert call(dt=0) == EUNSUPPORTED and "bf16" in err()
    assert call(do=None) == EINVAL and "do is NULL" in err()
    assert call(dg=None) == EINVAL
    assert call(ws_bytes=100) == EINVAL and "workspace" in err()
    assert call(ws=MIS) == EINVAL


def test_backward_varlen_rejects(lib):
    err = lambda: lib.gdr_last_error().decode()  # noqa: E731
    # as the fixed-length form, for tokens / 64 + N = 3 chunk slots (N = 2
    # sequences, 100 tokens, H = 3)
    chunks = 100 // 64 + 2
    st = chunks * 3 * 128 * 128 * 4
    rec = chunks * 3 * (3 * 64 * 128 * 2 + 64 * 64 * 2 + 128 * 4)
    fwd_gdn = (512 + 256 + chunks * 3 * 5888 + 255) // 256 * 256
    assert lib.gdr_backward_varlen_workspace_bytes(1, 2, 100, 3, 128, 128) == 2 * st + 512 + 256 + rec
    assert lib.gdr_backward_varlen_workspace_bytes(0, 2, 100, 3, 128, 128) == \
        2 * st + fwd_gdn + rec
    assert lib.gdr_backward_varlen_workspace_bytes(1, 2, 0, 3, 128, 128) == 0

    def call(dt=1, N=2, T_total=100, ws_bytes=1 << 30, cu=FAKE, host=None, **kw):
        hp = None
        if host is not None:
            arr = (ctypes.c_int32 * len(host))(*host)
            hp = ctypes.cast(arr, ctypes.c_void_p)
            call.keep = arr
        return lib.gdr_backward_chunked_varlen(
            dt, 1, N, T_total, 3, 128, 128, 64, F(1.0), cu, hp, FAKE, FAKE, FAKE, FAKE, FAKE,
            None, kw.get("do", FAKE), None, FAKE, FAKE, FAKE, FAKE, FAKE, None,
            kw.get("ws", FAKE), ws_bytes, None)
    assert call(dt=0) == EUNSUPPORTED and "bf16" in err()
    assert call(cu=None) == EINVAL and "cu_seqlens" in err()
    assert call(host=[0, 60, 40]) == EINVAL and "decreases" in err()
    assert call(host=[0, 40, 90]) == EINVAL and "T_total" in err()
    assert call(host=[1, 40, 100]) == EINVAL
    assert call(do=None) == EINVAL and "do is NULL" in err()
    assert call(ws_bytes=100) == EINVAL and "workspace" in err()
    assert call(N=0) == 0


def test_prefill_noalloc_rejects(lib):
    """The no-allocation prefill refuses, before any HIP call, a call whose
    workspace would not fit the library's own array, and bad arguments."""
    hdr = open(HEADER).read()
    m = re.search(r"#define GDR_NOALLOC_MAX_BYTES \(\(size_t\)(\d+) << (\d+)\)", hdr)
    assert m and int(m.group(1)) << int(m.group(2)) == gdr.NOALLOC_MAX_BYTES
    err = lambda: lib.gdr_last_error().decode()  # noqa: E731

    def call(dt=1, gk=0, B=1, T=64, H=1, D=128, chunk=64):
        return lib.gdr_prefill_chunked_noalloc(dt, gk, B, T, H, D, D, chunk, F(1.0), FAKE,
                                               FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, None)
    # GDN: 5888 bytes per (chunk, head); 4 x 4096 tokens x 64 heads is 98 MB
    need = gdr.workspace_bytes(torch.bfloat16, False, 4, 4 * 4096, 64)
    assert need > gdr.NOALLOC_MAX_BYTES
    assert call(B=4, T=4096, H=64) == EUNSUPPORTED and "beyond the library's own" in err()
    assert call(dt=7) == EINVAL and "dtype" in err()
    assert call(H=0) == EINVAL and "bad sizes" in err()
    assert call(D=96) == EUNSUPPORTED
    # the headline GDN workload fits
    assert gdr.workspace_bytes(torch.bfloat16, False, 4, 4 * 4096, 16) <= gdr.NOALLOC_MAX_BYTES


def test_binding_fails_loudly_without_library(tmp_path, monkeypatch):
    monkeypatch.setattr(gdr, "_LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(gdr, "_lib", None)
    with pytest.raises(gdr.GdrError, match="not built"):
        gdr.version()
