"""Parity metric shared by the GPU tests.

err(g, o) = max |g - o| / max |o|  (infinity-norm-wise relative error of one
tensor), the reading of "max relative error" used throughout: an
element-wise relative error is undefined where the oracle value is ~0.
"""
import numpy as np


def rel_err(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    den = np.max(np.abs(ref))
    if den == 0:
        return float(np.max(np.abs(got)))
    return float(np.max(np.abs(got - ref)) / den)


def assert_close(name, got, ref, tol):
    e = rel_err(got, ref)
    assert e <= tol, f"{name}: rel err {e:.3e} > {tol:.1e}"
    return e
