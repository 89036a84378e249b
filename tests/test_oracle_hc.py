"""Pins for the oracle's fused RMSNorm + Q8_0 down read and the up read.

Closed forms (constant R), invariances that fix where rs and w_norm enter
(R scaled by a power of two leaves lo unchanged; w_norm scaled scales lo),
and exact rational brute force on a tiny shape.
"""
import math
from fractions import Fraction

import numpy as np

from gemm_q8_amd import synth
from oracle.hc import hc_down, hc_up
from oracle.numerics import bf16_bits, bf16_to_f32, fp16_to_f32
from oracle.q8 import q8_0_gemv, quantize_q8_0

EPS = 1e-6


def _down_blocks(N=6, K=128, seed=0):
    return quantize_q8_0(synth.normal_f32(seed, "pin.hc.w", (N, K), 0.0, 0.02))


def test_down_constant_rows_closed_form():
    K = 128
    b = _down_blocks(K=K)
    c = 1.5
    R = np.full((2, K), bf16_bits(np.float32(c)), np.uint16)
    R[1] = bf16_bits(np.float32(-0.25))
    ones = np.full(K, bf16_bits(np.float32(1.0)), np.uint16)
    lo, rs, _ = hc_down(R, ones, b, EPS)
    d = fp16_to_f32(b.d).astype(np.float64)
    rowsum = (d * b.q.astype(np.int64).sum(axis=2)).sum(axis=1)       # sum_k d q
    for t, v in enumerate((c, -0.25)):
        want_rs = 1.0 / math.sqrt(v * v + EPS)
        assert abs(rs[t] - want_rs) <= 1e-15 * want_rs
        assert np.allclose(lo[t], want_rs * v * rowsum, rtol=1e-13, atol=0)


def test_down_rs_uses_R_and_is_applied_after_the_dot():
    b = _down_blocks()
    R = synth.bf16_normal(3, "pin.hc.R", (3, 128))
    wn = synth.bf16_normal(3, "pin.hc.wn", (128,), 1.0, 0.1)
    lo, rs, _ = hc_down(R, wn, b, EPS)
    R4 = bf16_bits(bf16_to_f32(R) * np.float32(4.0))          # exact power-of-two scaling
    lo4, rs4, _ = hc_down(R4, wn, b, EPS)
    assert np.allclose(rs4 * 4.0, rs, rtol=1e-6)               # eps is negligible here
    assert np.allclose(lo4, lo, rtol=1e-6, atol=0)
    wn2 = bf16_bits(bf16_to_f32(wn) * np.float32(2.0))
    lo2, rs2, _ = hc_down(R, wn2, b, EPS)
    assert np.array_equal(rs2, rs)                            # w_norm does not enter rs
    assert np.allclose(lo2, 2.0 * lo, rtol=1e-13, atol=0)


def test_down_with_unit_norm_weight_is_rmsnorm_then_gemv():
    b = _down_blocks()
    R = synth.bf16_normal(4, "pin.hc.R1", (2, 128))
    ones = np.full(128, bf16_bits(np.float32(1.0)), np.uint16)
    lo, rs, _ = hc_down(R, ones, b, EPS)
    y, _ = q8_0_gemv(b, bf16_to_f32(R))
    Rf = bf16_to_f32(R).astype(np.float64)
    want_rs = 1.0 / np.sqrt((Rf * Rf).mean(axis=1) + EPS)
    assert np.allclose(rs, want_rs, rtol=1e-14)
    assert np.allclose(lo, want_rs[:, None] * y, rtol=1e-12, atol=1e-15)


def test_down_brute_force_rational():
    N, K = 3, 64
    b = _down_blocks(N=N, K=K, seed=5)
    R = synth.bf16_normal(5, "pin.hc.Rb", (2, K))
    wn = synth.bf16_normal(5, "pin.hc.wnb", (K,), 1.0, 0.1)
    lo, rs, S = hc_down(R, wn, b, EPS)
    Rf, wf = bf16_to_f32(R), bf16_to_f32(wn)
    for t in range(2):
        ss = sum(Fraction(float(r)) ** 2 for r in Rf[t])
        r_t = 1.0 / math.sqrt(float(ss / K) + EPS)
        for n in range(N):
            acc = Fraction(0)
            for k in range(K):
                acc += (Fraction(float(fp16_to_f32(b.d[n, k // 32]))) * int(b.q[n, k // 32, k % 32])
                        * Fraction(float(Rf[t, k])) * Fraction(float(wf[k])))
            assert abs(r_t * float(acc) - lo[t, n]) <= 1e-12 * S[t, n]


def test_up_is_gemv_of_bf16_input():
    b = quantize_q8_0(synth.normal_f32(6, "pin.hc.up", (40, 64), 0.0, 0.02))
    lo = synth.bf16_normal(6, "pin.hc.lo", (3, 64))
    out, S = hc_up(lo, b)
    for k in (0, 33):
        e = np.zeros((1, 64), np.uint16)
        e[0, k] = bf16_bits(np.float32(1.0))
        o, _ = hc_up(e, b)
        assert np.array_equal(o[0], fp16_to_f32(b.d[:, k // 32]).astype(np.float64) * b.q[:, k // 32, k % 32])
    assert out.shape == (3, 40) and np.all(S >= np.abs(out))


# ---- the same reads on BF16 weights

def _pow2_blocks(N, K, seed):
    """Q8_0 blocks whose scales are powers of two: every weight d q is then a bf16 value."""
    b = quantize_q8_0(synth.normal_f32(seed, "pin.hc.p2", (N, K), 0.0, 0.02))
    d = fp16_to_f32(b.d)
    d2 = (2.0 ** np.round(np.log2(np.where(d > 0, d, 1.0)))).astype(np.float32)
    return b._replace(d=(d2.astype(np.float16)).view(np.uint16))


def _as_bf16_weights(blocks):
    w = (fp16_to_f32(blocks.d)[:, :, None] * blocks.q.astype(np.float32)).reshape(blocks.q.shape[0], -1)
    bits = bf16_bits(w)
    assert np.array_equal(bf16_to_f32(bits), w)                  # exact: d = 2^e, |q| <= 127
    return bits


def test_bf16_reads_equal_the_q8_reads_on_the_same_weights():
    """Two different weight decoders (Q8_0 blocks, bf16 bit patterns) describing the same real
    weights give the same down and up reads."""
    from oracle.hc import hc_down_bf16, hc_up_bf16
    b = _pow2_blocks(5, 96, seed=7)
    W = _as_bf16_weights(b)
    R = synth.bf16_normal(7, "pin.hc.R7", (3, 96))
    wn = synth.bf16_normal(7, "pin.hc.wn7", (96,), 1.0, 0.1)
    lo_q, rs_q, S_q = hc_down(R, wn, b, EPS)
    lo_b, rs_b, S_b = hc_down_bf16(R, wn, W, EPS)
    assert np.array_equal(rs_q, rs_b)
    assert np.allclose(lo_b, lo_q, rtol=1e-13, atol=1e-300) and np.allclose(S_b, S_q, rtol=1e-13)
    bu = _pow2_blocks(40, 64, seed=8)
    lo = synth.bf16_normal(8, "pin.hc.lo8", (2, 64))
    out_q, Sq = hc_up(lo, bu)
    out_b, Sb = hc_up_bf16(lo, _as_bf16_weights(bu))
    assert np.allclose(out_b, out_q, rtol=1e-13, atol=1e-300) and np.allclose(Sb, Sq, rtol=1e-13)


def test_bf16_down_brute_force_rational():
    from oracle.hc import hc_down_bf16
    N, K = 3, 64
    W = synth.bf16_normal(9, "pin.hc.Wb", (N, K), 0.0, 0.02)
    R = synth.bf16_normal(9, "pin.hc.Rbb", (2, K))
    wn = synth.bf16_normal(9, "pin.hc.wnbb", (K,), 1.0, 0.1)
    lo, rs, S = hc_down_bf16(R, wn, W, EPS)
    Rf, wf, Wf = bf16_to_f32(R), bf16_to_f32(wn), bf16_to_f32(W)
    for t in range(2):
        ss = sum(Fraction(float(r)) ** 2 for r in Rf[t])
        r_t = 1.0 / math.sqrt(float(ss / K) + EPS)
        assert abs(rs[t] - r_t) <= 1e-15 * r_t
        for n in range(N):
            acc = sum(Fraction(float(Wf[n, k])) * Fraction(float(Rf[t, k])) * Fraction(float(wf[k]))
                      for k in range(K))
            assert abs(r_t * float(acc) - lo[t, n]) <= 1e-12 * S[t, n]


def test_bf16_up_one_hot_picks_a_weight_column():
    from oracle.hc import hc_up_bf16
    W = synth.bf16_normal(10, "pin.hc.Wu", (24, 64), 0.0, 0.02)
    for k in (0, 31, 63):
        e = np.zeros((1, 64), np.uint16)
        e[0, k] = bf16_bits(np.float32(1.0))
        o, S = hc_up_bf16(e, W)
        assert np.array_equal(o[0], bf16_to_f32(W[:, k]).astype(np.float64))
        assert np.array_equal(S[0], np.abs(o[0]))


def test_pending_write_closed_forms_and_ties():
    """R' = R + P rounded once to bf16: P = 0 gives R; R = -P gives 0; sums of small integers are
    exact; 1 + 2^-8 is a tie between 1 and 1 + 2^-7 (even: 1); 1 + 3 * 2^-8 is a tie between
    1 + 2^-7 and 1 + 2^-6 (even: 1 + 2^-6); -0 + -0 is -0 and -0 + 0 is +0."""
    from oracle.hc import pending_write
    from oracle.numerics import bf16_bits
    f = lambda v: bf16_bits(np.array(v, np.float32))                         # noqa: E731
    R = f([[1.5, -3.0, 7.0, 1.0, 1.0, -0.0, -0.0, 100.0]])
    P = f([[0.0, 3.0, 5.0, 2.0 ** -8, 3 * 2.0 ** -8, -0.0, 0.0, -36.0]])
    want = f([[1.5, 0.0, 12.0, 1.0, 1.0 + 2.0 ** -6, -0.0, 0.0, 64.0]])
    assert pending_write(R, P).tolist() == want.tolist()


def test_pending_write_is_the_once_rounded_exact_sum():
    """Against exact rational sums rounded to nearest-even bf16 by hand (8-bit significands), over
    random bf16 pairs whose exponents differ by up to 30 (so the fp32 sum is sometimes inexact)."""
    from fractions import Fraction
    from oracle.hc import pending_write
    g = np.random.default_rng(5)
    n = 4000
    e1 = g.integers(-20, 20, n)
    e2 = e1 - g.integers(-30, 30, n)
    m1 = g.integers(128, 256, n) * g.choice([-1, 1], n)
    m2 = g.integers(128, 256, n) * g.choice([-1, 1], n)
    r = (m1 * np.ldexp(1.0, e1 - 7)).astype(np.float32)
    p = (m2 * np.ldexp(1.0, e2 - 7)).astype(np.float32)
    Rb = (r.view(np.uint32) >> 16).astype(np.uint16)
    Pb = (p.view(np.uint32) >> 16).astype(np.uint16)
    got = bf16_to_f32(pending_write(Rb[None], Pb[None])[0]).astype(np.float64)

    def rne_bf16(x):
        if x == 0:
            return Fraction(0)
        sgn = -1 if x < 0 else 1
        a = abs(x)
        e = 0
        while a >= 2:
            a /= 2
            e += 1
        while a < 1:
            a *= 2
            e -= 1
        m = a * 128                                   # 7 fraction bits
        lo = m.numerator // m.denominator
        rem = m - lo
        if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and lo % 2 == 1):
            lo += 1
        return sgn * Fraction(lo, 128) * Fraction(2) ** e
    for i in range(n):
        exact = Fraction(float(r[i])) + Fraction(float(p[i]))
        assert Fraction(float(got[i])) == rne_bf16(exact), i
