"""Helpers shared by the tests: conversions to the oracle's numpy inputs and error metrics.

Tolerances (row-normwise relative error on outputs, absolute error on alpha):
bf16 inputs with fp32 accumulation: 2e-3 and 1e-3; fp32 inputs: 1e-5 and 1e-5.
Indices, counts and scores: bit-exact."""
import numpy as np
import torch

TOL = {torch.bfloat16: (2e-3, 1e-3), torch.float32: (1e-5, 1e-5)}


def to_np(t: torch.Tensor):
    """CPU numpy view for the oracle: float32 as is, bf16 as uint16 bit patterns."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float32:
        return t.numpy()
    if t.dtype == torch.int32:
        return t.numpy()
    raise TypeError(t.dtype)


def sig_np(t: torch.Tensor):
    return t.detach().cpu().contiguous().numpy().view(np.uint32)


def row_rel_err(x, ref):
    """max over rows of ||x - ref||_2 / ||ref||_2 (rows = all but the last axis)."""
    x = np.asarray(x, np.float64).reshape(-1, np.shape(ref)[-1])
    r = np.asarray(ref, np.float64).reshape(-1, np.shape(ref)[-1])
    num = np.linalg.norm(x - r, axis=1)
    den = np.linalg.norm(r, axis=1)
    den = np.where(den == 0, 1.0, den)
    return float(np.max(num / den)) if num.size else 0.0


def alpha_err(a, ref):
    a = np.asarray(a, np.float64)
    ref = np.asarray(ref, np.float64)
    both_inf = np.isneginf(a) & np.isneginf(ref)
    d = np.where(both_inf, 0.0, np.abs(a - ref))
    return float(np.max(d)) if d.size else 0.0


def assert_close(out, alpha, ref_out, ref_alpha, dtype, what=""):
    tol_o, tol_a = TOL[dtype]
    out = out.detach().cpu().numpy() if isinstance(out, torch.Tensor) else out
    eo = row_rel_err(out, ref_out)
    assert np.all(np.isfinite(out)), "%s: non-finite output" % what
    assert eo <= tol_o, "%s: output row-relative error %.3e > %.1e" % (what, eo, tol_o)
    if alpha is not None:
        alpha = alpha.detach().cpu().numpy() if isinstance(alpha, torch.Tensor) else alpha
        ea = alpha_err(alpha, ref_alpha)
        assert ea <= tol_a, "%s: alpha abs error %.3e > %.1e" % (what, ea, tol_a)
        return eo, ea
    return eo, None
