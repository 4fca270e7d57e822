"""Parity tolerances, chosen by the output's storage type.

fp32 outputs:  |got - ref| <= 1e-6 + 1e-5 * |ref|
bf16 outputs:  |got - ref| <= 2^-7 * |ref| + 1e-3

The bf16 bound admits a one-unit-in-the-last-place disagreement at any
magnitude (a bf16 ulp is at most 2^-7 of the value), which is what fp32
intermediate arithmetic against a double-precision reference can produce.
"""
import numpy as np

FP32_ATOL = 1e-6
FP32_RTOL = 1e-5
BF16_ATOL = 1e-3
BF16_RTOL = 2.0 ** -7


def as_f64(a):
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def err_over_tol(got, ref, kind):
    """max over elements of |got - ref| / tol(ref); <= 1 passes."""
    g = as_f64(got)
    r = as_f64(ref)
    if kind == "f32":
        tol = FP32_ATOL + FP32_RTOL * np.abs(r)
    elif kind == "bf16":
        tol = BF16_ATOL + BF16_RTOL * np.abs(r)
    else:
        raise ValueError(kind)
    if g.size == 0:
        return 0.0
    return float(np.max(np.abs(g - r) / tol))


def assert_close(got, ref, kind, what=""):
    g = as_f64(got)
    r = as_f64(ref)
    assert g.shape == r.shape, f"{what}: shape {g.shape} vs {r.shape}"
    e = err_over_tol(g, r, kind)
    if not e <= 1.0:
        idx = np.unravel_index(np.argmax(np.abs(g - r)), g.shape)
        raise AssertionError(f"{what}: max err/tol = {e:.3f} at {idx}: got {g[idx]!r} ref {r[idx]!r}")
    return e


def ulp_f32(x):
    x = np.abs(np.asarray(x, dtype=np.float32))
    return np.spacing(x).astype(np.float64)
