"""Helpers shared by the tests: conversions to the oracle's numpy inputs and error metrics.

Tolerances (row-normwise relative error on outputs, absolute error on alpha):
bf16 inputs with fp32 accumulation: 2e-3 and 1e-3; fp32 inputs: 1e-5 and 1e-5.
Elementwise, no output element may be off by more than 5 x the normwise bound
times its row's RMS (1e-2 and 5e-5): the normwise bound alone would let one
element of a 128-wide row carry most of the row's error budget.
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


def elem_err(x, ref):
    """max over elements of |x - ref| / rms(ref's row) (rows = all but the last axis)."""
    x = np.asarray(x, np.float64).reshape(-1, np.shape(ref)[-1])
    r = np.asarray(ref, np.float64).reshape(-1, np.shape(ref)[-1])
    rms = np.sqrt(np.mean(r * r, axis=1))
    rms = np.where(rms == 0, 1.0, rms)
    return float(np.max(np.abs(x - r) / rms[:, None])) if x.size else 0.0


def alpha_err(a, ref):
    """max |a - ref|, where both -inf (an empty set) counts as equal: the -inf pairs are masked before the
    subtraction, which would give nan for them."""
    a = np.asarray(a, np.float64)
    ref = np.asarray(ref, np.float64)
    both_inf = np.isneginf(a) & np.isneginf(ref)
    d = np.abs(np.where(both_inf, 0.0, a) - np.where(both_inf, 0.0, ref))
    return float(np.max(d)) if d.size else 0.0


def assert_close(out, alpha, ref_out, ref_alpha, dtype, what=""):
    """Checks out (and alpha) against the oracle's values; prints the row-relative, elementwise and alpha errors
    (shown by pytest -s or on a failure) and returns (row-relative error, alpha error)."""
    tol_o, tol_a = TOL[dtype]
    out = out.detach().cpu().numpy() if isinstance(out, torch.Tensor) else out
    assert np.all(np.isfinite(out)), "%s: non-finite output" % what
    eo = row_rel_err(out, ref_out)
    ee = elem_err(out, ref_out)
    ea = None
    if alpha is not None:
        alpha = alpha.detach().cpu().numpy() if isinstance(alpha, torch.Tensor) else alpha
        ea = alpha_err(alpha, ref_alpha)
    print("%s: row-relative %.3e, elementwise %.3e, alpha %s" % (what, eo, ee, "-" if ea is None else "%.3e" % ea))
    assert eo <= tol_o, "%s: output row-relative error %.3e > %.1e" % (what, eo, tol_o)
    assert ee <= 5 * tol_o, "%s: output elementwise error %.3e x row RMS > %.1e" % (what, ee, 5 * tol_o)
    if alpha is not None:
        assert ea <= tol_a, "%s: alpha abs error %.3e > %.1e" % (what, ea, tol_a)
    return eo, ea
