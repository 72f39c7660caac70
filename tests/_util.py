"""Shared test helpers (no attention arithmetic here)."""
import numpy as np


def err_report(x, ref, tol):
    """Element-wise check: an element passes when |x - r| <= tol or
    |x - r| <= tol * |r|.  Returns (ok, max_abs_err, max_rel_err, n_bad)."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert x.shape == ref.shape, (x.shape, ref.shape)
    both_inf = np.isinf(x) & np.isinf(ref) & (np.sign(x) == np.sign(ref))
    d = np.where(both_inf, 0.0, np.abs(x - ref))
    d = np.where(np.isnan(d), np.inf, d)
    rel = d / np.maximum(np.abs(np.where(np.isinf(ref), 1.0, ref)), 1e-30)
    bad = ~((d <= tol) | (d <= tol * np.abs(ref)))
    return (not bad.any()), float(d.max(initial=0.0)), float(rel.max(initial=0.0)), int(bad.sum())


def assert_close(name, x, ref, tol):
    ok, ea, er, nb = err_report(x, ref, tol)
    assert ok, f"{name}: {nb} elements outside tol {tol} (max abs {ea:.3e}, max rel {er:.3e})"
    return ea, er
