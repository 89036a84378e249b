"""W8A8 decode product (oracle; test infrastructure).

W8A8 page, operator statement at the top: int8 x_q[M, K] times int8 W[K, N]
accumulates into int32; the int32 result is multiplied by the per-row
activation scale x_scale[M] and the per-column weight scale w_scale[N] and
written as bf16[M, N].

Readings:
  * the epilogue is read left to right in fp32: bf16( (fp32(acc) * x_scale[m]) * w_scale[n] ),
    two separately rounded fp32 products (no fused multiply-add), every rounding
    to nearest even;
  * int32 addition is exact here (|acc| <= 127*127*K < 2**31 for K <= 133,143),
    so the accumulator has exactly one correct value whatever the summation
    order (the page's "exact int32 order" matters only for determinism).
The accumulator is computed in int64 and checked to fit int32.
"""
from __future__ import annotations

import numpy as np

from .numerics import bf16_bits, bf16_to_f32, f32, round_half_away


def w8a8_acc(xq, W):
    """acc[m, n] = sum_k xq[m, k] * W[k, n], exact (int64, asserted to fit int32)."""
    acc = np.asarray(xq, dtype=np.int64) @ np.asarray(W, dtype=np.int64)
    assert np.all(np.abs(acc) < 2 ** 31), "accumulator leaves int32"
    return acc


def acc_to_f32(acc):
    """The epilogue's first step: the int32 accumulator as the nearest fp32, ties to even (above
    2^24 not every integer is an fp32)."""
    return np.asarray(acc, dtype=np.int64).astype(np.float32)


def w8a8_epilogue(acc, x_scale, w_scale):
    """bf16 bits of (fp32(acc) * x_scale[m]) * w_scale[n], each product rounded in fp32."""
    a = acc_to_f32(acc)
    v = (a * f32(x_scale)[:, None]).astype(np.float32)
    v = (v * f32(w_scale)[None, :]).astype(np.float32)
    return bf16_bits(v)


def w8a8_gemm(xq, x_scale, W, w_scale):
    """Returns (acc int64 [M, N], out bf16 bits [M, N])."""
    acc = w8a8_acc(xq, W)
    return acc, w8a8_epilogue(acc, x_scale, w_scale)


def quantize_per_token(x_bits):
    """Per-token int8 of a bf16 activation [M, K] (bit patterns): the x_q and x_scale the W8A8
    operator takes, made on the device ahead of the product (the W8A8 page times the product
    without it). The page fixes only the form (int8 per element, one fp32 scale per row);
    reading: symmetric in the row's largest magnitude, all in fp32 --
      amax = max_k |x[m, k]|,  x_scale = amax / 127,  inv = 127 / amax  (0 when amax = 0),
      x_q = clamp(round_half_away(x * inv), -127, 127)
    (one rounded division per row, then one rounded product per element). Returns (x_q int8
    [M, K], x_scale float32 [M])."""
    x = bf16_to_f32(x_bits).astype(np.float32)
    amax = np.max(np.abs(x), axis=1).astype(np.float32) if x.shape[1] else np.zeros(x.shape[0], np.float32)
    xs = f32(amax / np.float32(127))
    pos = amax > 0
    inv = np.where(pos, f32(np.float32(127) / np.where(pos, amax, np.float32(1))), np.float32(0))
    q = round_half_away(f32(x * f32(inv)[:, None]))
    return np.clip(q, -127, 127).astype(np.int8), xs
