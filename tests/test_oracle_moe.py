"""Pins for the oracle's routing, expert plan and routed-expert forward."""
import math

import numpy as np

from gemm_q8_amd import synth
from oracle.moe import expert_rows, moe_forward, plan, route
from oracle.q8 import dequantize, quantize_q8_0, quantize_q8_1_bf16


def test_route_closed_forms():
    ids, p = route(np.zeros((2, 16), np.float32), 4)
    assert ids.tolist() == [[0, 1, 2, 3]] * 2                  # ties go to the lower id
    assert np.allclose(p, 1 / 16, rtol=1e-15)
    l = np.log(np.array([[1.0, 2.0, 3.0, 0.5]], np.float64)).astype(np.float32)
    ids, p = route(l, 2)
    assert ids.tolist() == [[2, 1]]
    tot = 6.5
    assert abs(p[0, 0] - 3 / tot) < 1e-7 and abs(p[0, 1] - 2 / tot) < 1e-7


def test_route_matches_brute_force_sort():
    logits = synth.moe_inputs(T=4, E=512)["logits"]
    ids, p = route(logits, 8)
    for t in range(4):
        order = sorted(range(512), key=lambda e: (-float(logits[t, e]), e))[:8]
        assert ids[t].tolist() == order
        z = sum(math.exp(float(v) - float(logits[t].max())) for v in logits[t])
        for j in range(8):
            assert abs(p[t, j] - math.exp(float(logits[t, ids[t, j]]) - float(logits[t].max())) / z) < 1e-12


def test_plan_covers_every_entry_once():
    ids = np.array([[5, 1, 9], [1, 7, 5], [3, 2, 1]])
    pl = plan(ids)
    assert [e for e, _ in pl] == [1, 2, 3, 5, 7, 9]
    seen = sorted(i for _, es in pl for i in es)
    assert seen == list(range(9))
    for e, es in pl:
        assert es == sorted(es) and all(ids.flat[i] == e for i in es)


def _tiny_expert(e, D=64, F=32):
    w = synth.moe_expert_weights(e, D=D, F=F, seed=7)
    return quantize_q8_0(w["gate_up"]), quantize_q8_0(w["down"])


def test_expert_rows_match_dequantized_math():
    D, F = 64, 32
    x81 = quantize_q8_1_bf16(synth.bf16_normal(7, "pin.moe.x", (2, D)))
    gu, dn = _tiny_expert(3)
    xd = dequantize(x81)                                        # d_x * q_x as float64
    gu_v = dequantize(gu) @ xd[1]
    g, u = gu_v[:F], gu_v[F:]
    h = g * u / (1.0 + np.exp(-g))
    want = dequantize(dn) @ h
    r, S = expert_rows(x81, 1, gu, dn)
    assert np.allclose(r, want, rtol=1e-12, atol=1e-15)
    assert np.all(S >= np.abs(r))


def test_forward_is_weighted_sum_and_linear_in_weights():
    D, F = 64, 32
    x81 = quantize_q8_1_bf16(synth.bf16_normal(8, "pin.moe.x2", (2, D)))
    ids = np.array([[3, 1], [1, 4]])
    p = np.array([[0.6, 0.4], [0.25, 0.75]])
    blocks = lambda e: _tiny_expert(e, D, F)  # noqa: E731
    y, S = moe_forward(x81, ids, p, blocks)
    for t in range(2):
        want = sum(p[t, j] * expert_rows(x81, t, *blocks(ids[t, j]))[0] for j in range(2))
        assert np.allclose(y[t], want, rtol=1e-13, atol=1e-16)
    y2, _ = moe_forward(x81, ids, 2 * p, blocks)
    assert np.allclose(y2, 2 * y, rtol=1e-13, atol=1e-16)
    # one expert with weight one is that expert's rows
    y1, _ = moe_forward(x81, np.array([[4], [4]]), np.ones((2, 1)), blocks)
    assert np.allclose(y1[0], expert_rows(x81, 0, *blocks(4))[0], rtol=0, atol=0)


def test_requantized_h_within_the_dequantization_bound():
    """The q8_1(h) variant: every value of the down read's input moves by at most half its block's
    scale (plus the fp32 rounding of h), so each output row moves by at most
    sum_k |w_k| (d_blk(k) / 2 + |h_k| 2^-24); the variant reads each block's own scale."""
    from oracle.moe import requantize_h
    from oracle.numerics import fp16_to_f32
    D, F = 64, 96
    x81 = quantize_q8_1_bf16(synth.bf16_normal(9, "pin.moe.x3", (1, D)))
    gu, dn = _tiny_expert(5, D, F)
    r0, _ = expert_rows(x81, 0, gu, dn)
    rq, Sq = expert_rows(x81, 0, gu, dn, h_q8_1=True)
    gu_v = dequantize(gu) @ dequantize(x81)[0]
    g, u = gu_v[:F], gu_v[F:]
    h = g * u / (1.0 + np.exp(-g))
    hq = requantize_h(h)
    d = fp16_to_f32(quantize_q8_0(h.astype(np.float32)[None, :]).d[0]).astype(np.float64)
    dk = np.repeat(d, 32)
    assert np.all(np.abs(hq - h) <= dk / 2 * (1 + 2.0 ** -10) + np.abs(h) * 2.0 ** -24)
    W = dequantize(dn)
    bound = np.abs(W) @ (dk / 2 * (1 + 2.0 ** -10) + np.abs(h) * 2.0 ** -24)
    assert np.all(np.abs(rq - r0) <= bound * (1 + 1e-12))
    assert np.any(rq != r0)                                     # it is a different read
    assert np.allclose(rq, W @ hq, rtol=1e-13, atol=0) and np.all(Sq >= np.abs(rq))
    # each block's values are its own scale times integers in [-127, 127]
    k = np.rint(hq / dk)
    assert np.array_equal(hq, k * dk) and np.max(np.abs(k)) <= 127
    assert np.all(np.max(np.abs(k.reshape(-1, 32)), axis=1)[d > 0] == 127)


def test_requantized_forward_passes_the_flag_through():
    D, F = 64, 32
    x81 = quantize_q8_1_bf16(synth.bf16_normal(10, "pin.moe.x4", (2, D)))
    ids = np.array([[3, 1], [1, 4]])
    p = np.array([[0.6, 0.4], [0.25, 0.75]])
    blocks = lambda e: _tiny_expert(e, D, F)  # noqa: E731
    yq, _ = moe_forward(x81, ids, p, blocks, h_q8_1=True)
    for t in range(2):
        want = sum(p[t, j] * expert_rows(x81, t, *blocks(ids[t, j]), h_q8_1=True)[0] for j in range(2))
        assert np.allclose(yq[t], want, rtol=1e-13, atol=1e-16)


def test_expert_rows_gate_up_split_and_silu_closed_forms():
    """One 32-column block, hand-built so every dot product is one exact term: x is the one-hot
    q8_1 block (q = e_0, d = 1), gate/up row n holds d_n * e_0, and the down weight is the
    identity (row m = e_m, d = 1), so the routed row is h itself. Gate rows are 0..F-1 and up rows
    F..2F-1 (h = SiLU(g) * u with SiLU(g) = g * sigma(g)); the expected values are closed forms:
      sigma(0) = 1/2 so SiLU(0) = 0;  sigma(ln 3) = 3/4;  sigma(-ln 3) = 1/4;  SiLU(40) = 40 to
      1e-16.  g = fp16(ln 3) misses ln 3 by |delta| < 2^-11, and |SiLU'| < 1.1 there.
    Swapping the gate and up halves, or taking sigma(g) * u (no factor g), fails every case with
    g != u; dropping u fails the u = 0 rows."""
    from oracle.numerics import fp16_bits, fp16_to_f32
    from oracle.q8 import Q81Blocks, Q8Blocks
    F = D = 32
    one = fp16_bits(np.float32(1.0))
    xq = np.zeros((1, 1, 32), np.int8)
    xq[0, 0, 0] = 1
    x81 = Q81Blocks(d=np.array([[one]], np.uint16), s=np.array([[one]], np.uint16), q=xq)
    ln3 = float(np.log(3.0))
    # (g, u) per row n; rows 6.. are zero
    gu_vals = [(0.0, 2.0), (ln3, 2.0), (-ln3, 2.0), (40.0, 0.5), (-40.0, 0.5), (ln3, 0.0)]
    gd = np.zeros((2 * F, 1), np.uint16)
    gq = np.zeros((2 * F, 1, 32), np.int8)
    for n, (g, u) in enumerate(gu_vals):
        for row, v in ((n, g), (F + n, u)):
            gd[row, 0] = fp16_bits(np.float32(abs(v)))
            gq[row, 0, 0] = 1 if v >= 0 else -1
    gu = Q8Blocks(d=gd, q=gq)
    dq = np.zeros((D, 1, 32), np.int8)
    dq[np.arange(D), 0, np.arange(D)] = 1
    dn = Q8Blocks(d=np.full((D, 1), one, np.uint16), q=dq)
    r, S = expert_rows(x81, 0, gu, dn)
    g_ln3 = float(fp16_to_f32(fp16_bits(np.float32(ln3))))
    delta = abs(g_ln3 - ln3)
    assert 0 < delta < 2.0 ** -11
    assert r[0] == 0.0                                          # SiLU(0) = 0
    assert abs(r[1] - ln3 * 0.75 * 2.0) <= 1.1 * delta * 2.0     # ln 3 * 3/4 * u
    assert abs(r[2] - (-ln3) * 0.25 * 2.0) <= 1.1 * delta * 2.0  # -ln 3 * 1/4 * u
    assert abs(r[3] - 40.0 * 0.5) <= 1e-13                      # SiLU(40) = 40
    assert abs(r[4]) <= 1e-15                                   # SiLU(-40) ~ -1.7e-16
    assert r[5] == 0.0 and np.all(r[6:] == 0.0)                  # u = 0, or nothing routed
    assert np.array_equal(S, np.abs(r))                           # one term per output
