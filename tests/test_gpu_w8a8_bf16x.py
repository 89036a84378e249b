"""GPU parity of the W8A8 product on a bf16 activation: the per-token quantize kernel and the
bf16-activation product (one kernel up to 8 rows and 16384 values, else the quantize kernel
then the int8 product) give x_q / x_scale bit-exact against the oracle's per-token reading, and bf16 outputs
bit-exact against the oracle product on those x_q / x_scale, for M = 1..32, ragged N and K, the
full workload shapes, ties, zero rows, K = 0, staging in the workspace and graph replay."""
import numpy as np
import pytest
import torch

from gemm_q8_amd import synth
from gemm_q8_amd.device import to_dev, to_host, workspace
from oracle.numerics import bf16_bits
from oracle.w8a8 import quantize_per_token, w8a8_gemm

pytestmark = pytest.mark.gpu


def _pack(gpu, W):
    K, N = W.shape
    wp = torch.empty(gpu.gq8_w8a8_packed_bytes(K, N), dtype=torch.int8, device="cuda")
    gpu.gq8_w8a8_pack(to_dev(W), K, N, wp)
    return wp


def _quantize(gpu, x):
    M, K = x.shape
    xq = torch.full((M, K), 99, dtype=torch.int8, device="cuda")
    xs = torch.full((M,), 7.0, dtype=torch.float32, device="cuda")
    gpu.gq8_quantize_per_token(to_dev(x), M, K, xq, xs)
    torch.cuda.synchronize()
    return to_host(xq), to_host(xs)


def _fused(gpu, x, wp, w_scale, N, outs=True):
    M, K = x.shape
    out = torch.full((M, N), 0x7F7F, dtype=torch.int16, device="cuda")
    xq = torch.full((M, K), 99, dtype=torch.int8, device="cuda") if outs else None
    xs = torch.full((M,), 7.0, dtype=torch.float32, device="cuda") if outs else None
    nb = gpu.gq8_workspace_bytes(gpu.OP_W8A8_BF16X, M, N, K)
    assert (nb > 0) == (M > 8 or M * K > 16384)
    ws = workspace(nb) if not outs else None    # with both outputs given no workspace is needed
    gpu.gq8_w8a8_gemm_bf16x(to_dev(x), wp, to_dev(w_scale), out, xq, xs, M, N, K, ws,
                            0 if ws is None else nb)
    torch.cuda.synchronize()
    return to_host(out, np.uint16), (to_host(xq) if outs else None), (to_host(xs) if outs else None)


def _check(gpu, d, M, N, K, tag):
    xq_ref, xs_ref = quantize_per_token(d["x"])
    _, out_ref = w8a8_gemm(xq_ref, xs_ref, d["W"], d["w_scale"])
    xq, xs = _quantize(gpu, d["x"])
    assert np.array_equal(xq, xq_ref), f"quantize x_q {tag}"
    assert np.array_equal(xs.view(np.uint32), xs_ref.view(np.uint32)), f"quantize x_scale {tag}"
    out, xq2, xs2 = _fused(gpu, d["x"], _pack(gpu, d["W"]), d["w_scale"], N)
    assert np.array_equal(xq2, xq_ref), f"fused x_q {tag}"
    assert np.array_equal(xs2.view(np.uint32), xs_ref.view(np.uint32)), f"fused x_scale {tag}"
    assert np.array_equal(out, out_ref), f"fused out {tag}"


@pytest.mark.parametrize("M", [1, 2, 5, 8, 9, 16, 17, 32])
@pytest.mark.parametrize("N,K", [(48, 256), (37, 80), (160, 2048), (40, 2048 + 48), (160, 4096),
                                 (24, 8192), (40, 4352), (24, 6720)])
def test_bf16x_exact_small(gpu, M, N, K):
    d = synth.w8a8_bf16_inputs(M, N, K, seed=70 + M)
    _check(gpu, d, M, N, K, f"M={M} N={N} K={K}")


@pytest.mark.parametrize("M,N,K", [(16, 1536, 4096), (32, 2560, 4096), (1, 4096, 2048),
                                   (8, 4096, 2048), (4, 2560, 4096), (2, 64, 8192), (8, 64, 8192)])
def test_bf16x_full_size_exact(gpu, M, N, K):
    d = synth.w8a8_bf16_inputs(M, N, K, seed=5)
    _check(gpu, d, M, N, K, f"M={M} N={N} K={K}")


@pytest.mark.parametrize("M", [6, 20])
def test_bf16x_ties_zero_rows_and_outputs_optional(gpu, M):
    N, K = 32, 128
    d = synth.w8a8_bf16_inputs(M, N, K, seed=9)
    x = synth.bf16_bits_to_f32(d["x"]).copy()
    # row 0: amax 127 (inv = 1), exact half-integers -> ties away from zero
    x[0] = 0.0
    x[0, :8] = [127.0, 0.5, -0.5, 2.5, -2.5, 126.5, -126.5, 3.0]
    x[1] = 0.0                      # zero row: x_scale 0, quants 0
    x[2] = 0.0
    x[2, 77] = -3.0                 # one nonzero: it maps to -127
    x[M - 1] = 0.0                  # a zero last row
    d["x"] = bf16_bits(x)
    _check(gpu, d, M, N, K, "ties")
    xq_ref, xs_ref = quantize_per_token(d["x"])
    assert xq_ref[0, :8].tolist() == [127, 1, -1, 3, -3, 127, -127, 3]
    assert xs_ref[1] == 0 and not xq_ref[1].any() and xq_ref[2, 77] == -127
    # without the x_q / x_scale outputs the product is the same
    _, out_ref = w8a8_gemm(xq_ref, xs_ref, d["W"], d["w_scale"])
    out, _, _ = _fused(gpu, d["x"], _pack(gpu, d["W"]), d["w_scale"], N, outs=False)
    assert np.array_equal(out, out_ref)


def test_bf16x_zero_depth(gpu):
    M, N = 3, 40
    out = torch.full((M, N), 0x3F80, dtype=torch.int16, device="cuda")
    xs = torch.full((M,), 7.0, dtype=torch.float32, device="cuda")
    gpu.gq8_w8a8_gemm_bf16x(None, None, None, out, None, xs, M, N, 0, None, 0)
    xs2 = torch.full((M,), 7.0, dtype=torch.float32, device="cuda")
    gpu.gq8_quantize_per_token(None, M, 0, None, xs2)
    torch.cuda.synchronize()
    assert not out.any() and not xs.any() and not xs2.any()


@pytest.mark.parametrize("M,K", [(4, 4096), (16, 4096)])
def test_bf16x_graph_replay(gpu, M, K):
    N = 512
    d = synth.w8a8_bf16_inputs(M, N, K, seed=11)
    xq_ref, xs_ref = quantize_per_token(d["x"])
    _, out_ref = w8a8_gemm(xq_ref, xs_ref, d["W"], d["w_scale"])
    wp, x, wsc = _pack(gpu, d["W"]), to_dev(d["x"]), to_dev(d["w_scale"])
    out = torch.empty((M, N), dtype=torch.int16, device="cuda")
    xq = torch.empty((M, K), dtype=torch.int8, device="cuda")
    nb = gpu.gq8_workspace_bytes(gpu.OP_W8A8_BF16X, M, N, K)
    ws = workspace(nb)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        gpu.gq8_w8a8_gemm_bf16x(x, wp, wsc, out, xq, None, M, N, K, ws, nb, s)   # warm-up
        s.synchronize()
        with torch.cuda.graph(g, stream=s):
            gpu.gq8_w8a8_gemm_bf16x(x, wp, wsc, out, xq, None, M, N, K, ws, nb, s)
    for r in range(3):
        out.fill_(0x7F7F)
        xq.fill_(99)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(to_host(out, np.uint16), out_ref), f"replay {r}"
        assert np.array_equal(to_host(xq), xq_ref), f"replay {r}"
