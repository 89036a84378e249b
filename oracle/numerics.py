"""Number-format helpers for the oracle (test infrastructure; see package docstring).

fp16 conversion uses numpy's IEEE half type (round to nearest, ties to even).
bf16 has no numpy type: it is the top 16 bits of an fp32, rounded to nearest
with ties to even on the dropped 16 bits. Rounding to an integer is half away
from zero, as C's round() does (the rounding the Q8_0 quantizer on the HC-Q8
page names, via ggml).
"""
from __future__ import annotations

import numpy as np


def f32(x):
    return np.asarray(x, dtype=np.float32)


# ---------------------------------------------------------------- fp16 (IEEE binary16)

def fp16_bits(x):
    """fp32 -> fp16 bit patterns, round to nearest even."""
    return f32(x).astype(np.float16).view(np.uint16)


def fp16_to_f32(bits):
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float32)


# ---------------------------------------------------------------- bf16

def bf16_bits(x):
    """fp32 -> bf16 bit patterns, round to nearest even (NaN stays NaN)."""
    u = f32(x).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint16)
    nan = np.isnan(f32(x))
    if np.any(nan):
        r = np.where(nan, np.uint16(0x7FC0), r)
    return r


def bf16_to_f32(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_ulp(v):
    """Spacing of bf16 numbers in the binade of |v| (v float64 array); 0 -> smallest normal spacing."""
    a = np.abs(np.asarray(v, dtype=np.float64))
    a = np.where(a < 2.0 ** -126, 2.0 ** -126, a)
    e = np.floor(np.log2(a))
    return np.ldexp(1.0, (e - 7).astype(np.int64))


# ---------------------------------------------------------------- rounding

def round_half_away(v):
    """Round fp32 values to the nearest integer, ties away from zero (C round()).

    trunc(v) and v - trunc(v) are exact in fp32 for |v| < 2**23, so the tie test
    is exact; the result is returned as int64.
    """
    v = f32(v)
    t = np.trunc(v)
    frac = np.abs(v - t)  # exact
    up = frac >= np.float32(0.5)
    return (t.astype(np.int64) + np.where(up, np.sign(v).astype(np.int64), 0)).astype(np.int64)
