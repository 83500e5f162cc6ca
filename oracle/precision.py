"""Operand precision of the oracle's matrix products.

TEST INFRASTRUCTURE ONLY (see the oracle package header).

A configuration that runs its projections as bf16 GEMMs rounds each operand
of a matrix product to bfloat16 (8 significant bits, the fp32 exponent range)
and accumulates the products in a wider type.  With gemm="bf16" the oracle
does exactly that: both operands of every matrix product are rounded to the
nearest bf16 value (ties to even) and multiplied in f64.  With gemm="f64"
(the default everywhere) products are plain f64.  Every other step (the WKV
recurrence, norms, activations, elementwise ops) stays f64 in both modes.
"""
import numpy as np

GEMM_MODES = ("f64", "bf16")


def round_bf16(x):
    """Nearest value with 8 significant bits, ties to even; f64 in, f64 out.

    x = m 2^e with 0.5 <= |m| < 1 (frexp); m is rounded to a multiple of 2^-8
    by round-half-even (rint), which keeps 8 significant bits.  The values the
    tests use lie far inside the fp32 exponent range, so overflow and bf16
    subnormals do not arise.
    """
    x = np.asarray(x, np.float64)
    m, e = np.frexp(x)
    return np.ldexp(np.rint(m * 256.0) / 256.0, e)


def mm(a, b, gemm="f64"):
    """a @ b with the operand precision of `gemm` ("f64" or "bf16")."""
    if gemm == "bf16":
        return round_bf16(a) @ round_bf16(b)
    if gemm != "f64":
        raise ValueError(f"gemm must be one of {GEMM_MODES}, not {gemm!r}")
    return a @ b
