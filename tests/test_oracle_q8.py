"""Pins for the oracle's Q8_0 / q8_1 quantizers and the Q8_0 matrix-vector product.

Nothing here re-types the oracle's formulas: the checks are constructed blocks
with values known in closed form, the dequantization error bound, idempotence,
one-hot and block-indicator inputs, and exact rational brute force on tiny
shapes.
"""
from fractions import Fraction

import numpy as np

from gemm_q8_amd import synth
from oracle.numerics import bf16_to_f32, fp16_to_f32
from oracle.q8 import dequantize, q8_0_gemv, quantize_q8_0, quantize_q8_1_bf16, Q8Blocks


def _exact_block():
    # w_i = (i - 16) * 2^-7 with w_0 = -127 * 2^-7: amax = 127 * 2^-7, so d = 2^-7 exactly
    w = (np.arange(32, dtype=np.float32) - 16) * np.float32(2.0 ** -7)
    w[0] = -127 * 2.0 ** -7
    return w


def test_quantizer_exact_block():
    b = quantize_q8_0(_exact_block()[None, :])
    assert b.d[0, 0] == 0x2000                      # fp16 bits of 2^-7
    want = np.arange(32) - 16
    want[0] = -127
    assert b.q[0, 0].tolist() == want.tolist()


def test_quantizer_rounds_half_away_from_zero():
    w = np.zeros(32, dtype=np.float32)
    w[0] = 127 * 2.0 ** -7
    w[1], w[2], w[3], w[4] = 2.5 * 2.0 ** -7, -2.5 * 2.0 ** -7, 0.5 * 2.0 ** -7, 3.5 * 2.0 ** -7
    q = quantize_q8_0(w[None, :]).q[0, 0]
    assert q[:5].tolist() == [127, 3, -3, 1, 4]      # half-to-even would give 2, -2, 0, 4


def test_quantizer_zero_tiny_and_clamped_blocks():
    z = quantize_q8_0(np.zeros((1, 32), np.float32))
    assert z.d[0, 0] == 0 and not z.q.any()
    tiny = np.full((1, 32), 1e-9, np.float32)          # amax/127 underflows fp16 -> d = 0, q = 0
    t = quantize_q8_0(tiny)
    assert t.d[0, 0] == 0 and not t.q.any()
    # d32 = 1.49 * 2^-24 rounds to the fp16 subnormal 2^-24: amax/d = 189 -> clamped to 127
    w = np.zeros((1, 32), np.float32)
    w[0, 0] = np.float32(1.49 * 127 * 2.0 ** -24)
    w[0, 1] = -w[0, 0]
    c = quantize_q8_0(w)
    assert c.d[0, 0] == 0x0001
    assert c.q[0, 0, 0] == 127 and c.q[0, 0, 1] == -127


def test_dequant_error_bound_and_full_range():
    w = synth.normal_f32(0, "pin.w", (64, 256), 0.0, 0.02)
    b = quantize_q8_0(w)
    d = fp16_to_f32(b.d).astype(np.float64)
    err = np.abs(w.astype(np.float64).reshape(64, 8, 32) - d[:, :, None] * b.q)
    assert np.all(err <= d[:, :, None] * (0.5 + 2.0 ** -17))
    # every block with a normal fp16 scale uses the full quant range
    assert np.all(np.abs(b.q).max(axis=2) == 127)


def test_quantizer_is_idempotent():
    w = synth.normal_f32(0, "pin.idem", (16, 128), 0.0, 0.02)
    b = quantize_q8_0(w)
    b2 = quantize_q8_0(dequantize(b).astype(np.float32))
    assert np.array_equal(b.d, b2.d) and np.array_equal(b.q, b2.q)


def test_q8_1_sum_field():
    x = synth.bf16_normal(0, "pin.q81", (3, 96))
    b = quantize_q8_1_bf16(x)
    b0 = quantize_q8_0(bf16_to_f32(x))
    assert np.array_equal(b.d, b0.d) and np.array_equal(b.q, b0.q)
    s = fp16_to_f32(b.s).astype(np.float64)
    want = fp16_to_f32(b.d).astype(np.float64) * b.q.astype(np.int64).sum(axis=2)
    # s is d*sum(q) rounded once to fp16: relative error <= 2^-11
    assert np.all(np.abs(s - want) <= np.abs(want) * 2.0 ** -11 + 1e-30)


def test_gemv_one_hot_and_block_indicator():
    w = synth.normal_f32(0, "pin.gemv", (5, 96), 0.0, 0.02)
    b = quantize_q8_0(w)
    d = fp16_to_f32(b.d).astype(np.float64)
    q = b.q.astype(np.int64)
    for k in (0, 31, 32, 95):
        x = np.zeros((1, 96), np.float32)
        x[0, k] = 1.0
        y, _ = q8_0_gemv(b, x)
        assert np.array_equal(y[0], d[:, k // 32] * q[:, k // 32, k % 32])
    x = np.zeros((1, 96), np.float32)
    x[0, 32:64] = 1.0
    y, S = q8_0_gemv(b, x)
    assert np.array_equal(y[0], d[:, 1] * q[:, 1, :].sum(axis=1))
    assert np.array_equal(S[0], d[:, 1] * np.abs(q[:, 1, :]).sum(axis=1))


def test_gemv_brute_force_rational():
    T, N, K = 3, 4, 64
    w = synth.normal_f32(1, "pin.bf.w", (N, K), 0.0, 0.02)
    x = synth.normal_f32(1, "pin.bf.x", (T, K))
    b = quantize_q8_0(w)
    y, S = q8_0_gemv(b, x)
    for t in range(T):
        for n in range(N):
            acc = Fraction(0)
            for k in range(K):
                dn = Fraction(float(fp16_to_f32(b.d[n, k // 32])))
                acc += dn * int(b.q[n, k // 32, k % 32]) * Fraction(float(x[t, k]))
            assert abs(float(acc) - y[t, n]) <= 1e-12 * S[t, n]


def test_gemv_rows_are_independent():
    w = synth.normal_f32(2, "pin.rows.w", (7, 64), 0.0, 0.02)
    x = synth.normal_f32(2, "pin.rows.x", (4, 64))
    b = quantize_q8_0(w)
    y, _ = q8_0_gemv(b, x)
    for t in range(4):
        yt, _ = q8_0_gemv(b, x[t:t + 1])
        assert np.allclose(yt[0], y[t], rtol=0, atol=1e-15)
    # a block structure of one row only: Q8Blocks slicing keeps outputs
    yb, _ = q8_0_gemv(Q8Blocks(b.d[2:3], b.q[2:3]), x)
    assert np.allclose(yb[:, 0], y[:, 2], rtol=0, atol=1e-15)
