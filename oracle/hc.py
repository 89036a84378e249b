"""Fused RMSNorm + Q8_0 hyper-connection down read, and the Q8_0 up read (oracle; test infrastructure);
the same reads on BF16 weights (the reads the Q8_0 reads replace).

HC-Q8 page, "What changed": the down read works on R' * w_norm, unscaled, and
keeps the sums of squares; the RMSNorm factor rs is applied after the dot
product, when the partial sums are combined. The up read multiplies the Q8_0
up projection (its rows are K = 320 long) by the down read's output.

Readings taken where the page is not explicit:
  * rs is one value per token row over the whole row: rs = 1/sqrt(mean(R^2) + eps),
    eps = 1e-6, with the mean over the K columns of R (not of R * w_norm);
  * R' is R itself, or R + P rounded to bf16 when a pending write P is given (pending_write);
  * the down output lo is rs * dot, stored as bf16; rs is also returned;
  * the up read's own epilogue (pending write, gate, stream mean) is not
    defined on the page and is left out: the up output is the plain product,
    stored as bf16.
All arithmetic is float64; R * w_norm is exact there.
"""
from __future__ import annotations

import numpy as np

from .numerics import bf16_bits, bf16_to_f32
from .q8 import dequantize, q8_0_gemv


def _down(R_bits, wnorm_bits, W, eps):
    """The down read on real weights W [N, K] (float64): (lo, rs, S) as hc_down returns them."""
    R = bf16_to_f32(R_bits).astype(np.float64)
    wn = bf16_to_f32(wnorm_bits).astype(np.float64)
    K = R.shape[1]
    u = R * wn[None, :]
    ss = np.sum(R * R, axis=1)
    rs = 1.0 / np.sqrt(ss / K + eps)
    dot = u @ W.T
    lo = rs[:, None] * dot
    S = rs[:, None] * (np.abs(u) @ np.abs(W).T)
    return lo, rs, S


def pending_write(R_bits, P_bits):
    """The pending write (HC-Q8 page, "Summary": R_out, the pending write, is bitwise the default
    read's, written between the two reads; the page does not define it further). Reading: a
    pending residual update P is added to the stream before the down read, R' = R + P rounded to
    bf16 (to nearest, ties to even), and R' is both R_out and the down read's input. Two bf16
    values are added exactly in float64 here; rounding their sum to fp32 first gives the same
    bf16 (their fp32 sum is inexact only when the exponents differ by 16 or more, and then the
    smaller is below half a bf16 spacing of the larger). Returns bf16 bits [T, K]."""
    s = bf16_to_f32(R_bits).astype(np.float64) + bf16_to_f32(P_bits).astype(np.float64)
    return bf16_bits(s.astype(np.float32))


def hc_down(R_bits, wnorm_bits, blocks, eps=1e-6):
    """Down read.  R_bits bf16 [T, K], wnorm_bits bf16 [K], blocks: Q8_0 of W_down [N, K].

    Returns (lo [T, N], rs [T], S [T, N]) in float64, where S = rs * sum_k |d q u_k|
    is the scale of the pass rule.
    """
    return _down(R_bits, wnorm_bits, dequantize(blocks), eps)


def hc_up(lo_bits, blocks):
    """Up read.  lo_bits bf16 [T, K_lr], blocks: Q8_0 of W_up [N, K_lr].  Returns (out, S) float64."""
    return q8_0_gemv(blocks, bf16_to_f32(lo_bits))


# The same two reads on BF16 weights: the read the Q8_0 read replaces (HC-Q8 page, "Summary": the
# kernel-level BF16 -> Q8_0 times). Same readings as above; the weights are the bf16 values.

def hc_down_bf16(R_bits, wnorm_bits, W_bits, eps=1e-6):
    """Down read on W_down bf16 [N, K] (bit patterns).  Returns (lo, rs, S) as hc_down."""
    return _down(R_bits, wnorm_bits, bf16_to_f32(W_bits).astype(np.float64), eps)


def hc_up_bf16(lo_bits, W_bits):
    """Up read on W_up bf16 [N, K_lr]: out[t, n] = sum_k lo[t, k] W[n, k] in float64, and
    S = sum_k |lo W|.  Returns (out, S)."""
    x = bf16_to_f32(lo_bits).astype(np.float64)
    W = bf16_to_f32(W_bits).astype(np.float64)
    return x @ W.T, np.abs(x) @ np.abs(W).T
