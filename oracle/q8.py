"""Q8_0 / q8_1 block quantization and the Q8_0 matrix-vector product (oracle; test infrastructure).

Q8_0 (HC-Q8 page, "What changed"): a weight row is cut into blocks of 32
values; each block keeps 32 int8 quants and one fp16 scale (ggml's 34-byte
block). The quantizer the page names is ggml's: the scale is the block's
largest magnitude over 127, stored as fp16, and each quant is the value over
that scale rounded to an integer.

Readings taken where the page is not explicit:
  * the division w / d uses the stored fp16 scale (so scale and quants agree);
  * the amax / 127 quotient and the w / d quotient are fp32 operations (ggml's
    precision), and the fp16 store rounds to nearest even;
  * round() is C's round: half away from zero;
  * quants are clamped to [-127, 127] (only reachable when the scale is an fp16
    subnormal); a block whose fp16 scale is 0 gets all-zero quants.

The oracle keeps its own block structure -- scales d[N, K/32] (fp16 bits) and
quants q[N, K/32, 32] -- and never reads the library's split layout.

q8_1 (EP page, "What changed": the MoE input that is passed between cards is
"q8_1"): the page does not define the format. Reading: ggml's q8_1, i.e. the
Q8_0 quantizer above plus a per-block fp16 s = d * sum(q).
"""
from __future__ import annotations

from typing import NamedTuple

import numpy as np

from .numerics import f32, fp16_bits, fp16_to_f32, round_half_away, bf16_to_f32

BLOCK = 32


class Q8Blocks(NamedTuple):
    d: np.ndarray  # uint16 [rows, nblk]     fp16 bit patterns of the block scales
    q: np.ndarray  # int8   [rows, nblk, 32] quants


class Q81Blocks(NamedTuple):
    d: np.ndarray  # uint16 [rows, nblk]
    s: np.ndarray  # uint16 [rows, nblk]     fp16 of d * sum(q)
    q: np.ndarray  # int8   [rows, nblk, 32]


def quantize_q8_0(w):
    """Quantize fp32 rows w[N, K] (K % 32 == 0) into Q8_0 blocks."""
    w = f32(w)
    N, K = w.shape
    assert K % BLOCK == 0, "Q8_0 needs K to be a multiple of 32"
    blk = w.reshape(N, K // BLOCK, BLOCK)
    amax = np.max(np.abs(blk), axis=2)                       # fp32, exact
    d32 = (amax / np.float32(127.0)).astype(np.float32)       # fp32 quotient
    d_bits = fp16_bits(d32)                                   # stored scale
    d = fp16_to_f32(d_bits)                                   # its value, as fp32
    safe = np.where(d == 0, np.float32(1.0), d)
    v = (blk / safe[:, :, None]).astype(np.float32)           # fp32 quotient w / d
    q = np.clip(round_half_away(v), -127, 127)
    q = np.where((d == 0)[:, :, None], 0, q).astype(np.int8)
    return Q8Blocks(d=d_bits, q=q)


def quantize_q8_1_bf16(x_bits):
    """Quantize bf16 rows (bit patterns, [T, K]) into q8_1 blocks."""
    x = bf16_to_f32(x_bits)
    b = quantize_q8_0(x)
    qsum = b.q.astype(np.int64).sum(axis=2)
    # d (<= 11 significant bits) times |sum| <= 4064 (12 bits) is exact in fp32
    prod = (fp16_to_f32(b.d) * qsum.astype(np.float32)).astype(np.float32)
    return Q81Blocks(d=b.d, s=fp16_bits(prod), q=b.q)


def dequantize(blocks):
    """Real-valued weights d * q as float64 [rows, K] (exact: d*q fits an fp32 significand)."""
    d = fp16_to_f32(blocks.d).astype(np.float64)
    w = d[:, :, None] * blocks.q.astype(np.float64)
    return w.reshape(w.shape[0], -1)


def q8_0_gemv(blocks, x):
    """y[t, n] = sum_k d[n, k/32] * q[n, k] * x[t, k], in float64.

    Returns (y, S) with S[t, n] = sum_k |d q x|, the scale of the pass rule
    |y_gpu - y| <= 2e-3 * S used by the parity tests.
    """
    W = dequantize(blocks)
    xd = np.asarray(x, dtype=np.float64)
    y = xd @ W.T
    S = np.abs(xd) @ np.abs(W).T
    return y, S
