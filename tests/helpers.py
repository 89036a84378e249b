"""Shared pass rules for the GPU parity tests.

Q8_0 reads (fp32 accumulation): |y_gpu - y_ref| <= 2e-3 * S per output, S = sum_k |w_k x_k|
(the tolerance fixed for these reads). A bf16 output adds its own rounding: half a bf16 spacing
at the reference's magnitude (plus the tolerance), i.e. the GPU's fp32 value may round to either
neighbour when it sits near a rounding boundary.
"""
import numpy as np

from oracle.numerics import bf16_to_f32, bf16_ulp

REL = 2e-3


def check_f32(y_gpu, y_ref, S, what=""):
    y_gpu = np.asarray(y_gpu, dtype=np.float64)
    err = np.abs(y_gpu - y_ref)
    tol = REL * S
    bad = err > tol
    assert not bad.any(), (
        f"{what}: {bad.sum()} of {bad.size} outputs outside 2e-3*S; worst err/S = "
        f"{np.max(err / np.maximum(S, 1e-300)):.3e}")
    return float(np.max(err / np.maximum(S, 1e-300))) if err.size else 0.0


def check_bf16(bits_gpu, y_ref, S, what=""):
    v = bf16_to_f32(bits_gpu).astype(np.float64)
    err = np.abs(v - y_ref)
    tol = REL * S + 0.5 * bf16_ulp(np.abs(y_ref) + REL * S)
    bad = err > tol
    assert not bad.any(), (
        f"{what}: {bad.sum()} of {bad.size} bf16 outputs outside tolerance; worst err/tol = "
        f"{np.max(err / tol):.3e}")
    return float(np.max(err / tol)) if err.size else 0.0
