"""GPU parity over seeded random shapes within each entry point's limits (Q8_0 GEMV, the HC down
and up reads and the pair, W8A8 on int8 and on bf16 activations, the per-token quantizer, the
routed experts), each against the oracle at the same pass rules as the fixed-shape tests, plus
the zero-depth calls (outputs filled with zeros)."""
import numpy as np
import pytest
import torch

from gemm_q8_amd import synth
from gemm_q8_amd.device import q8_0_from_f32, to_dev, to_host, workspace
from oracle.hc import hc_down, hc_up
from oracle.moe import moe_forward, route
from oracle.q8 import q8_0_gemv, quantize_q8_0, quantize_q8_1_bf16
from oracle.w8a8 import quantize_per_token, w8a8_gemm
from tests.helpers import check_bf16, check_f32

pytestmark = pytest.mark.gpu


def _shapes(name, n, draw):
    g = np.random.default_rng(sum(map(ord, name)))
    return [draw(g) for _ in range(n)]


GEMV = _shapes("gemv", 10, lambda g: (int(g.integers(1, 17)), int(g.integers(1, 700)),
                                      32 * int(g.integers(1, 200))))
HC = _shapes("hc", 8, lambda g: (int(g.integers(1, 17)), 32 * int(g.integers(1, 33)),
                                 32 * int(g.integers(1, 400))))
# the tuned pair shapes (Nlr = 320: the whole-row down read with the fetch-ahead at T = 1, the
# combine inside the up read at T = 2..4, three kernels above) at random T and depth
HC320 = [(1, 320, 32 * 17), (1, 320, 32 * 389)] + _shapes(
    "hc320", 6, lambda g: (int(g.integers(1, 17)), 320, 32 * int(g.integers(1, 600))))
W8 = _shapes("w8a8", 10, lambda g: (int(g.integers(1, 33)), int(g.integers(1, 500)),
                                    16 * int(g.integers(1, 513))))


GEMV_FEW = _shapes("gemv-few", 8, lambda g: (int(g.integers(1, 4)), int(g.integers(1, 900)),
                                              32 * int(g.integers(1, 129))))
W8B = _shapes("w8a8-bf16x", 10, lambda g: (int(g.integers(1, 33)), int(g.integers(1, 500)),
                                           16 * int(g.integers(1, 513))))


def _moe_draw(g):
    T = int(g.integers(1, 17))
    topk = int(g.integers(1, min(16, 256 // T) + 1))
    E = int(g.integers(topk, 80))
    D = 32 * int(g.integers(1, 70))
    F = 32 * int(g.integers(1, 33))
    return T, E, topk, D, F


MOE = _shapes("moe", 8, _moe_draw)


@pytest.mark.parametrize("T,N,K", GEMV + GEMV_FEW)
def test_sweep_gemv(gpu, T, N, K):
    w = synth.normal_f32(60, "sweep.gemv.w", (N, K), 0.0, 0.02)
    x = synth.normal_f32(60, "sweep.gemv.x", (T, K))
    nb = gpu.gq8_workspace_bytes(gpu.OP_Q8_0_GEMV, T, N, K)
    y = torch.empty((T, N), dtype=torch.float32, device="cuda")
    gpu.gq8_q8_0_gemv(q8_0_from_f32(to_dev(w)), to_dev(x), y, T, N, K, workspace(nb), nb)
    torch.cuda.synchronize()
    y_ref, S = q8_0_gemv(quantize_q8_0(w), x)
    check_f32(to_host(y), y_ref, S, f"sweep gemv T={T} N={N} K={K}")


@pytest.mark.parametrize("T,Nlr,Khc", HC + HC320)
def test_sweep_hc_pair(gpu, T, Nlr, Khc):
    d = synth.hc_inputs(T, K=Khc, N=Nlr, seed=61)
    wd, wu = q8_0_from_f32(to_dev(d["w_down"])), q8_0_from_f32(to_dev(d["w_up"]))
    nb = gpu.gq8_workspace_bytes(gpu.OP_HC_PAIR, T, Nlr, Khc)
    lo = torch.empty((T, Nlr), dtype=torch.int16, device="cuda")
    rs = torch.empty((T,), dtype=torch.float32, device="cuda")
    out = torch.empty((T, Khc), dtype=torch.int16, device="cuda")
    gpu.gq8_hc_q8_pair(wd, to_dev(d["R"]), to_dev(d["w_norm"]), 1e-6, wu, lo, rs, out, T, Nlr, Khc,
                       workspace(nb), nb)
    torch.cuda.synchronize()
    lo_ref, rs_ref, S = hc_down(d["R"], d["w_norm"], quantize_q8_0(d["w_down"]))
    check_bf16(to_host(lo, np.uint16), lo_ref, S, f"sweep down T={T} Nlr={Nlr} Khc={Khc}")
    assert np.allclose(to_host(rs), rs_ref, rtol=1e-5, atol=0)
    out_ref, S_up = hc_up(to_host(lo, np.uint16), quantize_q8_0(d["w_up"]))
    check_bf16(to_host(out, np.uint16), out_ref, S_up, f"sweep up T={T} Nlr={Nlr} Khc={Khc}")


@pytest.mark.parametrize("M,N,K", W8)
def test_sweep_w8a8(gpu, M, N, K):
    d = synth.w8a8_inputs(M, N, K, seed=62)
    wp = torch.empty(gpu.gq8_w8a8_packed_bytes(K, N), dtype=torch.int8, device="cuda")
    gpu.gq8_w8a8_pack(to_dev(d["W"]), K, N, wp)
    nb = gpu.gq8_workspace_bytes(gpu.OP_W8A8, M, N, K)
    ws = workspace(nb)
    acc = torch.empty((M, N), dtype=torch.int32, device="cuda")
    out = torch.empty((M, N), dtype=torch.int16, device="cuda")
    xq = to_dev(d["xq"])
    gpu.gq8_w8a8_gemm_i32(xq, wp, acc, M, N, K, ws, nb)
    gpu.gq8_w8a8_gemm(xq, to_dev(d["x_scale"]), wp, to_dev(d["w_scale"]), out, M, N, K, ws, nb)
    torch.cuda.synchronize()
    acc_ref, out_ref = w8a8_gemm(d["xq"], d["x_scale"], d["W"], d["w_scale"])
    assert np.array_equal(to_host(acc), acc_ref), f"M={M} N={N} K={K}"
    assert np.array_equal(to_host(out, np.uint16), out_ref), f"M={M} N={N} K={K}"


@pytest.mark.parametrize("M,N,K", W8B)
def test_sweep_w8a8_bf16x(gpu, M, N, K):
    d = synth.w8a8_bf16_inputs(M, N, K, seed=64)
    wp = torch.empty(gpu.gq8_w8a8_packed_bytes(K, N), dtype=torch.int8, device="cuda")
    gpu.gq8_w8a8_pack(to_dev(d["W"]), K, N, wp)
    nb = gpu.gq8_workspace_bytes(gpu.OP_W8A8_BF16X, M, N, K)
    out = torch.empty((M, N), dtype=torch.int16, device="cuda")
    xq = torch.empty((M, K), dtype=torch.int8, device="cuda")
    xs = torch.empty((M,), dtype=torch.float32, device="cuda")
    x = to_dev(d["x"])
    gpu.gq8_w8a8_gemm_bf16x(x, wp, to_dev(d["w_scale"]), out, None, None, M, N, K, workspace(nb), nb)
    gpu.gq8_quantize_per_token(x, M, K, xq, xs)
    torch.cuda.synchronize()
    xq_ref, xs_ref = quantize_per_token(d["x"])
    _, out_ref = w8a8_gemm(xq_ref, xs_ref, d["W"], d["w_scale"])
    assert np.array_equal(to_host(xq), xq_ref), f"M={M} K={K}"
    assert np.array_equal(to_host(xs).view(np.uint32), xs_ref.view(np.uint32)), f"M={M} K={K}"
    assert np.array_equal(to_host(out, np.uint16), out_ref), f"M={M} N={N} K={K}"


@pytest.mark.parametrize("T,E,topk,D,F", MOE)
def test_sweep_moe(gpu, T, E, topk, D, F):
    seed = 63
    inp = synth.moe_inputs(T=T, E=E, D=D, seed=seed)
    ids_ref, p_ref = route(inp["logits"], topk)
    experts = lambda e: synth.moe_expert_weights(e, D=D, F=F, seed=seed)  # noqa: E731
    gu_b, dn_b = gpu.gq8_q8_0_bytes(2 * F, D), gpu.gq8_q8_0_bytes(D, F)
    agu = torch.full((E * gu_b,), 0x7F, dtype=torch.uint8, device="cuda")
    adn = torch.full((E * dn_b,), 0x7F, dtype=torch.uint8, device="cuda")
    for e in sorted(set(ids_ref.ravel().tolist())):
        w = experts(e)
        gpu.gq8_q8_0_quantize(to_dev(w["gate_up"]), 2 * F, D, agu[e * gu_b:(e + 1) * gu_b])
        gpu.gq8_q8_0_quantize(to_dev(w["down"]), D, F, adn[e * dn_b:(e + 1) * dn_b])
    ids = torch.empty((T, topk), dtype=torch.int32, device="cuda")
    wts = torch.empty((T, topk), dtype=torch.float32, device="cuda")
    gpu.gq8_moe_route(to_dev(inp["logits"]), T, E, topk, ids, wts)
    nb = gpu.gq8_moe_workspace_bytes(T, topk, D, F)
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    out = torch.empty((T, D), dtype=torch.int16, device="cuda")
    gpu.gq8_moe_q8_0_routed_bf16(to_dev(inp["x"]), ids, wts, agu, adn, out, T, topk, E, D, F, ws, nb)
    torch.cuda.synchronize()
    assert np.array_equal(to_host(ids), ids_ref)
    blocks = lambda e: (quantize_q8_0(experts(e)["gate_up"]), quantize_q8_0(experts(e)["down"]))  # noqa: E731
    y_ref, S = moe_forward(quantize_q8_1_bf16(inp["x"]), ids_ref, p_ref, blocks)
    check_bf16(to_host(out, np.uint16), y_ref, S, f"sweep moe T={T} E={E} topk={topk} D={D} F={F}")


def test_zero_depth_calls_fill_zeros(gpu):
    """K = 0 (an empty sum) writes zeros for the GEMV, the up read and W8A8."""
    y = torch.full((3, 17), 7.0, dtype=torch.float32, device="cuda")
    gpu.gq8_q8_0_gemv(None, None, y, 3, 17, 0, None, 0)
    out = torch.full((2, 40), 0x3F80, dtype=torch.int16, device="cuda")
    gpu.gq8_hc_q8_up(None, None, out, 2, 40, 0, None, 0)
    o8 = torch.full((4, 24), 0x3F80, dtype=torch.int16, device="cuda")
    gpu.gq8_w8a8_gemm(None, None, None, None, o8, 4, 24, 0, None, 0)
    torch.cuda.synchronize()
    assert not y.any() and not out.any() and not o8.any()
