"""Tolerance checks shared by the GPU parity tests.

The bars (written here, applied per tensor, outputs and final states
separately):
  * fp32 inputs: max |x - x_ref| <= 1e-4
  * bf16 inputs: ||x - x_ref||_F / ||x_ref||_F <= 2e-2
x_ref always comes from the fp64 oracle run on the stored input values.
"""
import numpy as np
import torch

FP32_MAX_ABS = 1e-4
BF16_REL_FRO = 2e-2


def to_np(t):
    if isinstance(t, torch.Tensor):
        return t.detach().float().cpu().numpy().astype(np.float64)
    return np.asarray(t, dtype=np.float64)


def rel_fro(x, ref):
    x, ref = to_np(x), to_np(ref)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(x - ref) / (den if den > 0 else 1.0))


def max_abs(x, ref):
    return float(np.abs(to_np(x) - to_np(ref)).max()) if np.size(ref) else 0.0


def assert_close(x, ref, dtype, what=""):
    """Apply the bar that belongs to the input dtype; returns the error."""
    if dtype == torch.float32:
        e = max_abs(x, ref)
        assert e <= FP32_MAX_ABS, "%s: max-abs %.3e > %.0e" % (what, e, FP32_MAX_ABS)
    else:
        e = rel_fro(x, ref)
        assert e <= BF16_REL_FRO, "%s: rel-Frobenius %.3e > %.0e" % (what, e, BF16_REL_FRO)
    assert np.all(np.isfinite(to_np(x))), "%s: non-finite values" % what
    return e


def announce(msg):
    print(msg, flush=True)
