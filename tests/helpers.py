"""Shared pass rules for the GPU parity tests.

Q8_0 reads (fp32 accumulation), two rules, both required:
  * per output: |y_gpu - y_ref| <= 2e-3 * S, S = sum_k |w_k x_k| (the tolerance fixed for these
    reads);
  * the HC-Q8 page's own parity figure ("What changed", its parity test): the read, against an
    fp64 reference computed from the same Q8_0 bytes, is within 1e-4 of the largest reference
    value: |y_gpu - y_ref| <= 1e-4 * max|y_ref|, the maximum taken over the whole output tensor
    (the plainest reading of "the largest value"). Unlike the first rule, it sees a single
    dropped or misread Q8_0 block, which moves an output by about 1e-2 of the largest value.
A bf16 output adds its own rounding to each rule: half a bf16 spacing at the reference's magnitude
(plus the tolerance), i.e. the GPU's fp32 value may round to either neighbour when it sits near a
rounding boundary.

Each check returns its worst ratios and records them (what, err/S, err/max|ref| and, for bf16
outputs, the error beyond half a bf16 spacing over max|ref|); with the
environment variable GQ8_PARITY_REPORT set to a path, the session writes the records there as JSON
lines (tests/conftest.py).
"""
import numpy as np

from oracle.numerics import bf16_to_f32, bf16_ulp

REL = 2e-3
PAGE_REL = 1e-4

RECORDS = []


def _ratios(err, y_ref, S):
    if err.size == 0:
        return 0.0, 0.0
    worst_s = float(np.max(err / np.maximum(S, 1e-300)))
    m = float(np.max(np.abs(y_ref)))
    worst_m = float(np.max(err) / m) if m > 0 else (0.0 if float(np.max(err)) == 0.0 else np.inf)
    return worst_s, worst_m


def _record(what, kind, worst_s, worst_m, page, excess_m=None):
    RECORDS.append({"case": what, "out": kind, "err_over_S": worst_s, "err_over_max": worst_m,
                    "excess_over_max": worst_m if excess_m is None else excess_m, "page_rule": page})
    extra = "" if excess_m is None else f", beyond half a bf16 spacing {excess_m:.3e}"
    print(f"[parity] {what}: worst err/S = {worst_s:.3e}, worst err/max|ref| = {worst_m:.3e}{extra}")


def check_f32(y_gpu, y_ref, S, what="", page=True):
    y_gpu = np.asarray(y_gpu, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    err = np.abs(y_gpu - y_ref)
    tol = REL * S
    bad = err > tol
    worst_s, worst_m = _ratios(err, y_ref, S)
    _record(what, "f32", worst_s, worst_m, page)
    assert not bad.any(), (
        f"{what}: {bad.sum()} of {bad.size} outputs outside 2e-3*S; worst err/S = {worst_s:.3e}")
    if page and err.size:
        assert worst_m <= PAGE_REL, (
            f"{what}: worst err / max|ref| = {worst_m:.3e} > 1e-4 (the HC-Q8 page's parity figure)")
    return worst_s


def check_bf16(bits_gpu, y_ref, S, what="", page=True):
    v = bf16_to_f32(bits_gpu).astype(np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    err = np.abs(v - y_ref)
    tol = REL * S + 0.5 * bf16_ulp(np.abs(y_ref) + REL * S)
    bad = err > tol
    worst_s, worst_m = _ratios(err, y_ref, S)
    m = float(np.max(np.abs(y_ref))) if err.size else 0.0
    excess = np.maximum(err - 0.5 * bf16_ulp(np.abs(y_ref)), 0.0)
    excess_m = float(np.max(excess) / m) if m > 0 else 0.0
    _record(what, "bf16", worst_s, worst_m, page, excess_m)
    assert not bad.any(), (
        f"{what}: {bad.sum()} of {bad.size} bf16 outputs outside tolerance; worst err/tol = "
        f"{np.max(err / tol):.3e}")
    if page and err.size:
        pt = PAGE_REL * float(np.max(np.abs(y_ref)))
        ptol = pt + 0.5 * bf16_ulp(np.abs(y_ref) + pt)
        pbad = err > ptol
        assert not pbad.any(), (
            f"{what}: {pbad.sum()} of {pbad.size} bf16 outputs farther than half a bf16 spacing "
            f"+ 1e-4 max|ref| from the reference (the HC-Q8 page's parity figure); worst "
            f"err/tol = {np.max(err / ptol):.3e}")
    return float(np.max(err / tol)) if err.size else 0.0
