"""GPU test of gdr_prefill_chunked_noalloc (the prefill that takes no
workspace and allocates nothing, for callers that cannot allocate): through
the C ABI, against gdr_prefill_chunked with a caller's workspace on the same
inputs, on two calls in a row on one GPU (the second smaller, so that it
reads the library's array after a larger call left its contents there), and
against the fp64 oracle at the bf16 bar."""
import ctypes

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
F = ctypes.c_float


def ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def both(lib, x, dt, gk):
    """(o, ht) from gdr_prefill_chunked with a workspace and from the
    no-allocation call, on the same inputs."""
    B, T, H, D = x["q"].shape
    stream = ctypes.c_void_p(torch.cuda.current_stream(DEV).cuda_stream)
    args = (x["q"], x["k"], x["v"], x["g"], x["beta"], x["h0"])
    o1, o2 = torch.empty_like(x["v"]), torch.full_like(x["v"], 3.0)
    h1 = torch.empty((B, H, D, D), device=DEV, dtype=torch.float32)
    h2 = torch.full_like(h1, 5.0)
    need = gdr.workspace_bytes(x["q"].dtype, gk == 1, B, B * T, H)
    ws = torch.empty(max(need, 1), device=DEV, dtype=torch.uint8)
    rc = lib.gdr_prefill_chunked(dt, gk, B, T, H, D, D, 64, F(1.0), *[ptr(t) for t in args],
                                 ptr(o1), ptr(h1), ptr(ws), need, stream)
    assert rc == 0, lib.gdr_last_error()
    rc = lib.gdr_prefill_chunked_noalloc(dt, gk, B, T, H, D, D, 64, F(1.0),
                                         *[ptr(t) for t in args], ptr(o2), ptr(h2), stream)
    assert rc == 0, lib.gdr_last_error()
    torch.cuda.synchronize(DEV)
    return (o1, h1), (o2, h2)


@pytest.mark.parametrize("gate", ["scalar", "channel"])
def test_noalloc_matches_the_workspace_call(gate):
    lib = gdr._load()
    gk = 1 if gate == "channel" else 0
    # two calls in a row, the second smaller; the second also has a gate of
    # zero in one token so that the channel gate's second pass runs
    for i, (B, T, H) in enumerate([(2, 300, 4), (1, 70, 2)]):
        announce("noalloc %s call %d: B=%d T=%d H=%d" % (gate, i, B, T, H))
        x = synthetic.prefill_inputs(B, T, H, 128, torch.bfloat16, gate, seed=90 + i, device=DEV)
        if i == 1:
            x["g"][:, 40] = float("-inf")
        (o1, h1), (o2, h2) = both(lib, x, 1, gk)
        assert torch.equal(o1, o2) and torch.equal(h1, h2)
        o_ref, ht_ref = oracle.forward(x["q"], x["k"], x["v"], x["g"], x["beta"], h0=x["h0"])
        assert_close(o2, o_ref, torch.bfloat16, "o")
        assert_close(h2, ht_ref, torch.bfloat16, "ht")


def test_noalloc_fp32_and_binding():
    """fp32 inputs need no workspace; the binding passes the caller's o and
    ht through."""
    x = synthetic.prefill_inputs(1, 50, 2, 64, torch.float32, "scalar", seed=95, device=DEV)
    o = torch.empty_like(x["v"])
    ht = torch.empty((1, 2, 64, 64), device=DEV, dtype=torch.float32)
    gdr.prefill_noalloc(x["q"], x["k"], x["v"], x["g"], x["beta"], o, h0=x["h0"], ht=ht)
    torch.cuda.synchronize(DEV)
    o_ref, ht_ref = oracle.forward(x["q"], x["k"], x["v"], x["g"], x["beta"], h0=x["h0"])
    assert_close(o, o_ref, torch.float32, "o")
    assert_close(ht, ht_ref, torch.float32, "ht")
