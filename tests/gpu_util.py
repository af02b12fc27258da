"""Tolerance checks shared by the GPU parity tests.

The bars (written here, applied per tensor, outputs and final states
separately):
  * fp32 inputs: max |x - x_ref| <= 1e-4
  * bf16 inputs: ||x - x_ref||_F / ||x_ref||_F <= 2e-2, and beside it every
    row (last axis: one token's output, one value row of a state) within
    5e-2 of its reference row, relative to that row's norm or to the
    tensor's RMS row norm, whichever is larger (a row that is small next to
    the others is judged on the tensor's scale: its error comes from
    rounding of operands of the tensor's size).  The whole-tensor bar alone
    cannot see one wrong row among thousands; this one sees any row whose
    error reaches a twentieth of a typical row.
x_ref always comes from the fp64 oracle run on the stored input values.
"""
import numpy as np
import torch

FP32_MAX_ABS = 1e-4
BF16_REL_FRO = 2e-2
BF16_ROW_REL = 5e-2


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


def row_rel(x, ref):
    """Largest relative error of a row (last axis) and its index; the
    denominator is the larger of the reference row's norm and the tensor's
    RMS row norm."""
    x, ref = to_np(x), to_np(ref)
    if ref.size == 0:
        return 0.0, 0
    x2 = x.reshape(-1, x.shape[-1])
    r2 = ref.reshape(-1, ref.shape[-1])
    rn = np.linalg.norm(r2, axis=1)
    floor = float(np.sqrt(np.mean(rn * rn)))
    err = np.linalg.norm(x2 - r2, axis=1) / np.maximum(rn, max(floor, 1e-30))
    i = int(np.argmax(err))
    return float(err[i]), i


def assert_close(x, ref, dtype, what="", rows=True):
    """Apply the bar that belongs to the input dtype; returns the error."""
    assert np.all(np.isfinite(to_np(x))), "%s: non-finite values" % what
    if dtype == torch.float32:
        e = max_abs(x, ref)
        assert e <= FP32_MAX_ABS, "%s: max-abs %.3e > %.0e" % (what, e, FP32_MAX_ABS)
    else:
        e = rel_fro(x, ref)
        assert e <= BF16_REL_FRO, "%s: rel-Frobenius %.3e > %.0e" % (what, e, BF16_REL_FRO)
        if rows:
            er, i = row_rel(x, ref)
            assert er <= BF16_ROW_REL, "%s: row %d relative error %.3e > %.0e" % (
                what, i, er, BF16_ROW_REL)
    return e


def announce(msg):
    print(msg, flush=True)


def assert_pairs_close(x, ref, what=""):
    """bf16 bar per (sequence, head): x and ref are [pairs, ...] (one entry
    per pair, any trailing shape); each pair's relative Frobenius error must
    meet the bar on its own.  Returns the largest."""
    x, ref = to_np(x), to_np(ref)
    worst = 0.0
    for i in range(ref.shape[0]):
        e = rel_fro(x[i], ref[i])
        assert e <= BF16_REL_FRO, "%s: pair %d rel-Frobenius %.3e > %.0e" % (what, i, e, BF16_REL_FRO)
        worst = max(worst, e)
    return worst


def heads_first(t):
    """[B, T, H, ...] -> [B * H, T, ...] (one entry per (sequence, head))."""
    t = to_np(t)
    B, T, H = t.shape[:3]
    return np.moveaxis(t, 2, 1).reshape(B * H, T, *t.shape[3:])
