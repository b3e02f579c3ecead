"""Comparison helpers for parity tests (test infrastructure)."""
import numpy as np


def slice_rel_err(x, y, cu=None):
    """Per (sequence, head) slice error max|x-y| / max|y| (absolute max|x-y| when max|y| = 0).

    x, y: outputs [T, H, dv] (slices are token ranges of ``cu`` per head) or states [N, H, dk, dv].
    Returns an array [N, H]."""
    x = np.asarray(x, np.float64)
    y = np.asarray(y, np.float64)
    assert x.shape == y.shape, (x.shape, y.shape)
    if x.ndim == 4:
        d = np.abs(x - y).max(axis=(2, 3))
        m = np.abs(y).max(axis=(2, 3))
    else:
        T, H = x.shape[:2]
        cu = np.asarray([0, T] if cu is None else cu)
        N = len(cu) - 1
        d = np.zeros((N, H))
        m = np.zeros((N, H))
        for n in range(N):
            a, b = int(cu[n]), int(cu[n + 1])
            if b > a:
                d[n] = np.abs(x[a:b] - y[a:b]).max(axis=(0, 2))
                m[n] = np.abs(y[a:b]).max(axis=(0, 2))
    return np.where(m > 0, d / np.where(m > 0, m, 1), d)


def assert_close(x, y, tol, cu=None, what=""):
    e = slice_rel_err(x, y, cu)
    worst = float(e.max()) if e.size else 0.0
    assert worst <= tol, f"{what}: max per-slice error {worst:.3e} > {tol:.1e} at {np.unravel_index(e.argmax(), e.shape)}"
    print(f"  {what}: max per-slice error {worst:.3e} (tol {tol:.0e})", flush=True)
    return worst
