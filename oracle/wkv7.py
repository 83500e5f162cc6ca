"""WKV7 recurrence oracle: numpy front end of ``wkv7_oracle.c`` (f64).

TEST INFRASTRUCTURE ONLY (see the package header).

The recurrence follows "Foundry/cuda_kernels/timemix.cu" (tm_fwd_device,
k_composites: the WKV7 call takes r, w, k', v', A=-kk, B=kk*a) and the per-head
WKV state-backward block of "infotheory .../rwkv7/model.rs"
(accumulate_token_step_gradients).  Per (b, h) and token t:

    sa   = S a_t                       (old state)
    S    = S diag(w_t) + sa b_t^T + v_t k_t^T
    y_t  = S r_t                       (updated state)

Arrays: token vectors [B][T][H][N], state [B][H][N][N] with S[i][j], i the
value index, j the key index.
"""
import ctypes
import os

import numpy as np

from . import build as _build

_lib = None


def _load():
    global _lib
    if _lib is None:
        path = _build.build(force=False)
        lib = ctypes.CDLL(path)
        dp = ctypes.POINTER(ctypes.c_double)
        lib.oracle_wkv7_forward.argtypes = [ctypes.c_int] * 4 + [dp] * 9
        lib.oracle_wkv7_forward.restype = ctypes.c_int
        lib.oracle_wkv7_backward.argtypes = [ctypes.c_int] * 4 + [dp] * 16
        lib.oracle_wkv7_backward.restype = ctypes.c_int
        lib.oracle_num_threads.argtypes = []
        lib.oracle_num_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def _f64(x):
    return None if x is None else np.ascontiguousarray(x, dtype=np.float64)


def _ptr(x):
    if x is None:
        return ctypes.POINTER(ctypes.c_double)()
    return x.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def num_threads() -> int:
    """OpenMP threads the oracle uses (OMP_NUM_THREADS or the host's cores)."""
    return int(_load().oracle_num_threads())


def forward(r, w, k, v, a, b, s0=None):
    """y [B][T][H][N] and S_T [B][H][N][N] of the recurrence, in f64.

    s0=None means a zero initial state.
    """
    r, w, k, v, a, b, s0 = map(_f64, (r, w, k, v, a, b, s0))
    B, T, H, N = r.shape
    for x in (w, k, v, a, b):
        assert x.shape == (B, T, H, N)
    if s0 is not None:
        assert s0.shape == (B, H, N, N)
    y = np.zeros((B, T, H, N))
    sT = np.zeros((B, H, N, N))
    rc = _load().oracle_wkv7_forward(B, T, H, N, _ptr(r), _ptr(w), _ptr(k), _ptr(v),
                                     _ptr(a), _ptr(b), _ptr(s0), _ptr(y), _ptr(sT))
    if rc != 0:
        raise MemoryError("oracle_wkv7_forward failed to allocate")
    return y, sT


def backward(r, w, k, v, a, b, dy, s0=None, dsT=None):
    """Gradients of L = <dy, y> + <dsT, S_T> with respect to every input.

    Returns dict with dr, dw, dk, dv, da, db ([B][T][H][N]) and ds0.
    """
    r, w, k, v, a, b, dy, s0, dsT = map(_f64, (r, w, k, v, a, b, dy, s0, dsT))
    B, T, H, N = r.shape
    out = {n: np.zeros((B, T, H, N)) for n in ("dr", "dw", "dk", "dv", "da", "db")}
    out["ds0"] = np.zeros((B, H, N, N))
    rc = _load().oracle_wkv7_backward(
        B, T, H, N, _ptr(r), _ptr(w), _ptr(k), _ptr(v), _ptr(a), _ptr(b),
        _ptr(s0), _ptr(dy), _ptr(dsT),
        _ptr(out["dr"]), _ptr(out["dw"]), _ptr(out["dk"]), _ptr(out["dv"]),
        _ptr(out["da"]), _ptr(out["db"]), _ptr(out["ds0"]))
    if rc != 0:
        raise MemoryError("oracle_wkv7_backward failed to allocate")
    return out


def step(r, w, k, v, a, b, state):
    """Single-token decode: r..b are [B][H][N]; returns (y [B][H][N], new state).

    Defined as the T=1 forward from the given state.
    """
    B, H, N = np.shape(r)
    rs = [np.asarray(x, dtype=np.float64).reshape(B, 1, H, N) for x in (r, w, k, v, a, b)]
    y, s1 = forward(*rs, s0=state)
    return y.reshape(B, H, N), s1
