"""Pins for the C++ oracle (oracle/c/gq8_oracle.cpp): its number formats against an independent
library (numpy's IEEE half, torch's bf16) at every half value and every rounding midpoint; its
quantizer byte for byte against the numpy oracle, plus the dequantization bound; its reads against
the numpy oracle (float64 sums in another order: within 1e-12 of S), one-hot exactness and an
exact rational brute force on tiny shapes; W8A8 bit for bit; and one thread bitwise equal to all
host cores (a fixed k-order per output)."""
from fractions import Fraction

import numpy as np
import pytest

from gemm_q8_amd import synth
from oracle import c_oracle as C
from oracle.hc import hc_down, hc_up
from oracle.moe import moe_forward, route
from oracle.numerics import bf16_to_f32, fp16_to_f32
from oracle.q8 import dequantize, q8_0_gemv, quantize_q8_0, quantize_q8_1_bf16
from oracle.w8a8 import w8a8_gemm


def test_f16_conversion_every_value_and_midpoint():
    """Every finite half value, and the midpoint (and its fp32 neighbours) between every pair of
    adjacent halves, converted by the C++ oracle and by numpy's IEEE half type."""
    h = np.arange(0, 0x7C00, dtype=np.uint32).astype(np.uint16)
    v = h.view(np.float16).astype(np.float64)
    mids = (v[:-1] + v[1:]) / 2                                 # exact in float64 and float32
    m32 = mids.astype(np.float32)
    up = np.nextafter(m32, np.float32(np.inf))
    dn = np.nextafter(m32, np.float32(0))
    x = np.concatenate([v.astype(np.float32), m32, up, dn, [65504, 65519.99, 65520, 1e9]]).astype(np.float32)
    x = np.concatenate([x, -x])
    want = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(C.f16_bits(x), want)


def test_bf16_conversion_against_torch():
    torch = pytest.importorskip("torch")
    g = np.random.default_rng(3)
    x = (g.standard_normal(100000) * 50).astype(np.float32)
    u = x.view(np.uint32).copy()
    u[:3000] = (u[:3000] & np.uint32(0xFFFF0000)) | np.uint32(0x8000)   # exact ties
    x = u.view(np.float32)
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(C.bf16_bits(x), want)


def test_quantizer_matches_numpy_oracle_and_dequant_bound():
    w = synth.normal_f32(50, "pin.c.q", (64, 1024), 0.0, 0.02)
    w[3, :32] = 0.0                                             # a zero block
    w[5, :32] = np.float32(1e-9)                                 # a block whose fp16 scale is 0
    w[7, 32:64] = (np.arange(32) - 16).astype(np.float32) * np.float32(0.5)   # ties of w / d
    a, b = C.quantize_q8_0(w), quantize_q8_0(w)
    assert np.array_equal(a.d, b.d) and np.array_equal(a.q, b.q)
    d = fp16_to_f32(a.d).astype(np.float64)
    err = np.abs(w.reshape(64, 32, 32) - d[:, :, None] * a.q)
    live = d > 0
    assert np.all((err <= d[:, :, None] * (0.5 + 2.0 ** -17))[live])
    # a block whose fp16 scale rounds to 0 (amax / 127 below half the smallest fp16 step) is zeros
    assert np.all(a.q[~live] == 0) and np.all(np.abs(w.reshape(64, 32, 32)[~live]) < 127 * 2.0 ** -25)


def _rel(a, b, S):
    return float(np.max(np.abs(a - b) / np.maximum(S, 1e-300)))


@pytest.mark.parametrize("T,N,K", [(1, 1024, 4096), (4, 37, 2080), (16, 8, 96)])
def test_gemv_matches_numpy_oracle(T, N, K):
    w = synth.normal_f32(51, "pin.c.g", (N, K), 0.0, 0.02)
    x = synth.normal_f32(51, "pin.c.gx", (T, K))
    b = quantize_q8_0(w)
    y, S = C.q8_0_gemv(b, x)
    y2, S2 = q8_0_gemv(b, x)
    assert _rel(y, y2, S2) <= 1e-12 and np.allclose(S, S2, rtol=1e-12, atol=0)
    y1, _ = C.q8_0_gemv(b, x, threads=1)
    assert np.array_equal(y, y1)                                 # one thread == all cores


def test_gemv_one_hot_and_rational_brute_force():
    N, K = 5, 64
    w = synth.normal_f32(52, "pin.c.oh", (N, K), 0.0, 0.02)
    b = quantize_q8_0(w)
    x = np.zeros((2, K), np.float32)
    x[0, 37] = 1.0
    x[1] = synth.normal_f32(52, "pin.c.ohx", (1, K))[0]
    y, _ = C.q8_0_gemv(b, x)
    assert np.array_equal(y[0], fp16_to_f32(b.d[:, 1]).astype(np.float64) * b.q[:, 1, 5])
    for n in range(N):
        exact = sum(Fraction(float(fp16_to_f32(b.d[n, k // 32]))) * int(b.q[n, k // 32, k % 32])
                    * Fraction(float(x[1, k])) for k in range(K))
        assert abs(Fraction(y[1, n]) - exact) <= abs(exact) * Fraction(1, 2 ** 45) + Fraction(1, 2 ** 80)


@pytest.mark.parametrize("T,N,K", [(1, 320, 16384), (6, 64, 1056)])
def test_hc_reads_match_numpy_oracle(T, N, K):
    d = synth.hc_inputs(T, K=K, N=N, seed=53)
    bd, bu = quantize_q8_0(d["w_down"]), quantize_q8_0(d["w_up"])
    lo, rs, S = C.hc_down(d["R"], d["w_norm"], bd)
    lo2, rs2, S2 = hc_down(d["R"], d["w_norm"], bd)
    assert _rel(lo, lo2, S2) <= 1e-12 and np.allclose(rs, rs2, rtol=1e-14, atol=0)
    lo1, rs1, _ = C.hc_down(d["R"], d["w_norm"], bd, threads=1)
    assert np.array_equal(lo, lo1) and np.array_equal(rs, rs1)
    lob = C.bf16_bits(lo.astype(np.float32))
    out, Su = C.hc_up(lob, bu)
    out2, Su2 = hc_up(lob, bu)
    assert _rel(out, out2, Su2) <= 1e-12


def test_hc_down_constant_rows_closed_form():
    """R = c everywhere, w_norm = 1: rs = 1 / sqrt(c^2 + eps) and lo = rs c sum_k d q."""
    N, K, c = 4, 512, 0.75
    w = synth.normal_f32(54, "pin.c.cf", (N, K), 0.0, 0.02)
    b = quantize_q8_0(w)
    R = np.full((1, K), 0x3F40, np.uint16)                        # bf16 0.75
    wn = np.full(K, 0x3F80, np.uint16)
    lo, rs, _ = C.hc_down(R, wn, b)
    assert rs[0] == 1.0 / np.sqrt(c * c + 1e-6)
    assert np.allclose(lo[0], rs[0] * c * dequantize(b).sum(axis=1), rtol=1e-13, atol=0)


@pytest.mark.parametrize("M,N,K", [(16, 1536, 4096), (3, 40, 64), (32, 17, 128)])
def test_w8a8_bitwise_numpy_oracle(M, N, K):
    dd = synth.w8a8_inputs(M, N, K)
    acc, out = C.w8a8_gemm(dd["xq"], dd["x_scale"], dd["W"], dd["w_scale"])
    acc2, out2 = w8a8_gemm(dd["xq"], dd["x_scale"], dd["W"], dd["w_scale"])
    assert np.array_equal(acc, acc2) and np.array_equal(out, out2)
    acc1, out1 = C.w8a8_gemm(dd["xq"], dd["x_scale"], dd["W"], dd["w_scale"], threads=1)
    assert np.array_equal(acc, acc1) and np.array_equal(out, out1)


def test_w8a8_epilogue_rounding_pins():
    """The epilogue cases whose bf16 output depends on the accumulator's rounding to fp32 (see
    the numpy oracle's pins): acc = 2^24 + 1 at x_scale = 1 + 2^-8 -> 0x4B80, and acc = 2^24 + 3 at
    the fp32 just below 1 + 2^-8 -> 0x4B81; acc = 257 and 259 at unit scales -> 256, 260."""
    xs_below = np.array([np.float32(1 + 2.0 ** -8).view(np.uint32) - 1], np.uint32).view(np.float32)[0]
    targets = [2 ** 24 + 1, 2 ** 24 + 3, 257, 259]
    from oracle.w8a8 import w8a8_epilogue
    accs = np.array([[t] for t in targets], np.int64)
    xs = np.array([1 + 2.0 ** -8, xs_below, 1.0, 1.0], np.float32)
    want = w8a8_epilogue(accs, xs, np.ones(1, np.float32))[:, 0].tolist()
    assert want == [0x4B80, 0x4B81, 0x4380, 0x4382]
    # the C++ epilogue on the same accumulators: x_q = 1 against W = acc needs |acc| <= 127, so
    # spread each accumulator over K columns of 127 plus a remainder
    for m, t in enumerate(targets):
        n127, rem = divmod(t, 127)
        Km = ((n127 + 1 + 15) // 16) * 16
        xr = np.zeros((1, Km), np.int8)
        xr[0, :n127 + 1] = 1
        Wc = np.zeros((Km, 1), np.int8)
        Wc[:n127, 0] = 127
        Wc[n127, 0] = rem
        acc, out = C.w8a8_gemm(xr, xs[m:m + 1], Wc, np.ones(1, np.float32))
        assert acc[0, 0] == t and out[0, 0] == want[m]


def test_moe_matches_numpy_oracle():
    T, E, topk, D, F = 4, 64, 8, 256, 64
    inp = synth.moe_inputs(T=T, E=E, D=D, seed=55)
    ids, p = route(inp["logits"], topk)
    x81 = quantize_q8_1_bf16(inp["x"])
    cache = {}

    def blocks(e):
        if e not in cache:
            w = synth.moe_expert_weights(e, D=D, F=F, seed=55)
            cache[e] = (quantize_q8_0(w["gate_up"]), quantize_q8_0(w["down"]))
        return cache[e]
    y, S = C.moe_forward(x81, ids, p, blocks)
    y2, S2 = moe_forward(x81, ids, p, blocks)
    assert _rel(y, y2, S2) <= 1e-12 and np.allclose(S, S2, rtol=1e-12, atol=0)
    y1, _ = C.moe_forward(x81, ids, p, blocks, threads=1)
    assert np.array_equal(y, y1)
