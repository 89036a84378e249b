"""Pins for the oracle's W8A8 product: integer brute force, closed forms, and rounding ties."""
import numpy as np

from gemm_q8_amd import synth
from oracle.numerics import bf16_to_f32
from oracle.w8a8 import w8a8_acc, w8a8_epilogue, w8a8_gemm


def test_acc_brute_force_python_ints():
    M, K, N = 3, 40, 5
    x = synth.int8_uniform(0, "pin.w8.x", (M, K))
    W = synth.int8_uniform(0, "pin.w8.W", (K, N))
    acc = w8a8_acc(x, W)
    for m in range(M):
        for n in range(N):
            assert acc[m, n] == sum(int(x[m, k]) * int(W[k, n]) for k in range(K))


def test_acc_closed_forms():
    K = 4096
    assert np.all(w8a8_acc(np.ones((2, K), np.int8), np.ones((K, 3), np.int8)) == K)
    big = np.full((1, K), 127, np.int8)
    assert w8a8_acc(big, np.full((K, 1), -127, np.int8))[0, 0] == -127 * 127 * K
    x = synth.int8_uniform(1, "pin.w8.neg", (4, 64))
    W = synth.int8_uniform(1, "pin.w8.negW", (64, 7))
    assert np.array_equal(w8a8_acc(-x.astype(np.int16), W), -w8a8_acc(x, W))
    # one-hot row / column pick single entries of W / x
    e = np.zeros((1, 64), np.int8)
    e[0, 17] = 1
    assert np.array_equal(w8a8_acc(e, W)[0], W[17].astype(np.int64))


def test_epilogue_ties_to_even():
    one = np.ones(1, np.float32)
    acc = np.array([[257, 259, 258, -257]])
    out = w8a8_epilogue(acc, one, np.ones(4, np.float32))
    assert out[0].tolist() == [0x4380, 0x4382, 0x4381, 0xC380]    # 256, 260, 258, -256


def test_epilogue_scales_rows_and_columns():
    acc = np.array([[1000, -2000], [3000, 4]])
    xs = np.array([0.5, 0.25], np.float32)
    ws = np.array([2.0, 4.0], np.float32)
    out = bf16_to_f32(w8a8_epilogue(acc, xs, ws))
    assert out.tolist() == [[1000.0, -4000.0], [1504.0, 4.0]]      # 1500 rounds to bf16 1504


def test_gemm_shapes_and_int32_range():
    d = synth.w8a8_inputs(16, 48, 256)
    acc, out = w8a8_gemm(d["xq"], d["x_scale"], d["W"], d["w_scale"])
    assert acc.shape == (16, 48) and out.shape == (16, 48) and out.dtype == np.uint16


# ---- per-token quantization of a bf16 activation

def test_per_token_quantization_bounds_and_extremes():
    from oracle.numerics import bf16_bits, bf16_to_f32
    from oracle.w8a8 import quantize_per_token
    x = synth.bf16_normal(20, "pin.w8.xq", (5, 256))
    q, xs = quantize_per_token(x)
    xf = bf16_to_f32(x).astype(np.float64)
    amax = np.max(np.abs(xf), axis=1)
    assert np.array_equal(xs, (amax / 127).astype(np.float32))
    # the largest magnitude of each row maps to +-127, every code is within the row's range
    for m in range(5):
        k = int(np.argmax(np.abs(xf[m])))
        assert abs(int(q[m, k])) == 127 and np.sign(q[m, k]) == np.sign(xf[m, k])
    # dequantization error: at most half a scale (plus the rounded products' slack)
    err = np.abs(q.astype(np.float64) * xs[:, None].astype(np.float64) - xf)
    assert np.all(err <= xs[:, None] * (0.5 + 1e-5))
    # a zero row: scale 0, quants 0; a row scaled by a power of two keeps its quants
    z, zs = quantize_per_token(np.zeros((1, 64), np.uint16))
    assert zs[0] == 0 and not z.any()
    x4 = bf16_bits(bf16_to_f32(x) * np.float32(4.0))
    q4, xs4 = quantize_per_token(x4)
    assert np.array_equal(q4, q) and np.array_equal(xs4, 4 * xs)


def test_per_token_quantization_ties_go_away_from_zero():
    from oracle.numerics import bf16_bits
    from oracle.w8a8 import quantize_per_token
    # amax = 127 makes inv = 1 exactly: x = j + 0.5 are exact ties
    row = np.array([127.0, 0.5, -0.5, 2.5, -2.5, 126.5, -126.5, 3.0], np.float32)
    q, xs = quantize_per_token(bf16_bits(row)[None, :])
    assert xs[0] == np.float32(1.0)
    assert q[0].tolist() == [127, 1, -1, 3, -3, 127, -127, 3]


def test_accumulator_to_fp32_rounds_to_nearest_even():
    """Above 2^24 the int32 accumulator is rounded to the nearest fp32, ties to even:
    2^24 + 1 -> 16777216, 2^24 + 3 -> 16777220 (not 16777218, which truncation gives), and at
    2^25 (spacing 4) 2^25 + 2 -> 2^25, 2^25 + 6 -> 2^25 + 8; below 2^24 every integer is exact."""
    from oracle.w8a8 import acc_to_f32
    acc = np.array([2 ** 24 + 1, 2 ** 24 + 3, -(2 ** 24 + 1), -(2 ** 24 + 3), 2 ** 25 + 2,
                    2 ** 25 + 6, 2 ** 24 - 1, 66064384, -66064383], np.int64)
    want = [16777216, 16777220, -16777216, -16777220, 2 ** 25, 2 ** 25 + 8, 2 ** 24 - 1,
            66064384, -66064384]
    assert acc_to_f32(acc).astype(np.int64).tolist() == want


def test_epilogue_sees_the_accumulator_rounding():
    """Cases where the bf16 output depends on how the accumulator became an fp32 (x_scale chosen
    so the scaled value lands on or next to a bf16 rounding boundary at 2^24 (1 + 2^-8)):
      acc = 2^24 + 1, x_scale = 1 + 2^-8: fp32(acc) = 2^24, times x_scale is exactly the bf16
        midpoint, which ties to even: 2^24 (0x4B80); an exact conversion would give 0x4B81;
      acc = 2^24 + 3, x_scale = the fp32 just below 1 + 2^-8: 16777220 * x_scale lies above the
        midpoint (0x4B81); a truncated 16777218 would land below it (0x4B80)."""
    xs_below = np.array([np.float32(1 + 2.0 ** -8).view(np.uint32) - 1], np.uint32).view(np.float32)
    out = w8a8_epilogue(np.array([[2 ** 24 + 1], [2 ** 24 + 3]], np.int64),
                        np.array([1 + 2.0 ** -8, xs_below[0]], np.float32), np.ones(1, np.float32))
    assert out[:, 0].tolist() == [0x4B80, 0x4B81]
