"""GPU parity of the W8A8 product: int32 accumulators and bf16 outputs bit-exact against the
oracle, for M = 1..32 (int8 MFMA; the VALU dot4 kernel forced where it exists, M <= 15),
ragged N and K, the full workload shapes, rounding ties, and graph replay."""
import numpy as np
import pytest
import torch

from gemm_q8_amd import synth
from gemm_q8_amd.device import to_dev, to_host, workspace
from oracle.w8a8 import w8a8_acc, w8a8_gemm

pytestmark = pytest.mark.gpu


def _pack(gpu, W):
    K, N = W.shape
    wp = torch.empty(gpu.gq8_w8a8_packed_bytes(K, N), dtype=torch.int8, device="cuda")
    gpu.gq8_w8a8_pack(to_dev(W), K, N, wp)
    return wp


def _run(gpu, d, M, N, K, i32=False):
    wp = _pack(gpu, d["W"])
    nb = gpu.gq8_workspace_bytes(gpu.OP_W8A8, M, N, K)
    ws = workspace(nb)
    xq = to_dev(d["xq"])
    if i32:
        acc = torch.empty((M, N), dtype=torch.int32, device="cuda")
        gpu.gq8_w8a8_gemm_i32(xq, wp, acc, M, N, K, ws, nb)
        return to_host(acc)
    out = torch.empty((M, N), dtype=torch.int16, device="cuda")
    gpu.gq8_w8a8_gemm(xq, to_dev(d["x_scale"]), wp, to_dev(d["w_scale"]), out, M, N, K, ws, nb)
    return to_host(out, np.uint16)


@pytest.mark.parametrize("M", [1, 2, 3, 4, 8, 15, 16, 17, 31, 32])
@pytest.mark.parametrize("N,K", [(48, 256), (37, 80), (160, 4096)])
def test_w8a8_exact_small(gpu, M, N, K):
    d = synth.w8a8_inputs(M, N, K, seed=30 + M)
    acc_ref, out_ref = w8a8_gemm(d["xq"], d["x_scale"], d["W"], d["w_scale"])
    assert np.array_equal(_run(gpu, d, M, N, K, i32=True), acc_ref)
    assert np.array_equal(_run(gpu, d, M, N, K), out_ref)


@pytest.mark.parametrize("M,N,K", [(16, 1536, 4096)] + [(m, 2560, 4096) for m in (1, 4, 8, 16, 32)]
                         + [(m, 4096, 2048) for m in (1, 4, 8, 16, 32)])
def test_w8a8_full_size_exact(gpu, M, N, K):
    d = synth.w8a8_inputs(M, N, K)
    acc_ref, out_ref = w8a8_gemm(d["xq"], d["x_scale"], d["W"], d["w_scale"])
    assert np.array_equal(_run(gpu, d, M, N, K, i32=True), acc_ref)
    assert np.array_equal(_run(gpu, d, M, N, K), out_ref)


@pytest.mark.parametrize("M", [1, 2, 4, 8, 15])
@pytest.mark.parametrize("N,K", [(37, 80), (160, 4096), (40, 8192)])
def test_w8a8_forced_kernels_exact(gpu, monkeypatch, M, N, K):
    """GQ8_W8A8_KERNEL=dot and =mfma force the VALU dot4 kernel and the int8 MFMA kernel where both
    exist (M <= 15): each is bit-exact against the oracle, so the choice between them is speed
    only."""
    d = synth.w8a8_inputs(M, N, K, seed=90 + M)
    acc_ref, out_ref = w8a8_gemm(d["xq"], d["x_scale"], d["W"], d["w_scale"])
    for kern in ("dot", "mfma"):
        monkeypatch.setenv("GQ8_W8A8_KERNEL", kern)
        assert np.array_equal(_run(gpu, d, M, N, K, i32=True), acc_ref), kern
        assert np.array_equal(_run(gpu, d, M, N, K), out_ref), kern


def test_w8a8_extreme_accumulators(gpu):
    M, N, K = 16, 32, 4096
    d = {"xq": np.full((M, K), 127, np.int8), "W": np.full((K, N), -127, np.int8),
         "x_scale": np.ones(M, np.float32), "w_scale": np.ones(N, np.float32)}
    d["xq"][1] = -127
    acc = _run(gpu, d, M, N, K, i32=True)
    assert acc[0, 0] == -127 * 127 * K and acc[1, 0] == 127 * 127 * K


def test_w8a8_rounding_ties(gpu):
    # acc = 257 and 259 with unit scales: bf16 ties go to even (256, 260)
    M, N, K = 2, 16, 64
    xq = np.zeros((M, K), np.int8)
    xq[0, :3] = [127, 127, 3]
    xq[1, :3] = [127, 127, 5]
    W = np.zeros((K, N), np.int8)
    W[:3, :] = 1
    d = {"xq": xq, "W": W, "x_scale": np.ones(M, np.float32), "w_scale": np.ones(N, np.float32)}
    out = _run(gpu, d, M, N, K)
    assert (out[0] == 0x4380).all() and (out[1] == 0x4382).all()


def test_w8a8_graph_replay_and_poison(gpu):
    M, N, K = 16, 1536, 4096
    d = synth.w8a8_inputs(M, N, K)
    wp = _pack(gpu, d["W"])
    nb = gpu.gq8_workspace_bytes(gpu.OP_W8A8, M, N, K)
    cb = gpu.gq8_workspace_counter_bytes(gpu.OP_W8A8, M, N, K)
    ws = workspace(nb)
    xq, xs, wsc = to_dev(d["xq"]), to_dev(d["x_scale"]), to_dev(d["w_scale"])
    out = torch.empty((M, N), dtype=torch.int16, device="cuda")
    gpu.gq8_w8a8_gemm(xq, xs, wp, wsc, out, M, N, K, ws, nb)
    torch.cuda.synchronize()
    ref = out.clone()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            gpu.gq8_w8a8_gemm(xq, xs, wp, wsc, out, M, N, K, ws, nb, s)
    for _ in range(3):
        out.zero_()
        if nb > cb:
            ws[cb:nb].fill_(0x5A)
        torch.cuda.synchronize()
        with torch.cuda.stream(s):
            g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref)
        if cb:
            assert int(ws[:cb].count_nonzero()) == 0


@pytest.mark.parametrize("M", [1, 16, 32])
def test_w8a8_max_depth(gpu, M):
    """K = 8192, the largest depth (16 waves x 8 k-steps of 64), exact against the oracle."""
    N, K = 80, 8192
    d = synth.w8a8_inputs(M, N, K, seed=3)
    acc_ref, out_ref = w8a8_gemm(d["xq"], d["x_scale"], d["W"], d["w_scale"])
    assert np.array_equal(_run(gpu, d, M, N, K, i32=True), acc_ref)
    assert np.array_equal(_run(gpu, d, M, N, K), out_ref)


@pytest.mark.parametrize("K", [4160, 4352, 5120, 6096, 6720, 7232, 8128])
@pytest.mark.parametrize("M,N", [(1, 40), (16, 48), (32, 40), (9, 2064)])
def test_w8a8_deep_ragged_steps(gpu, M, N, K):
    """Depths past 4096 whose k-step count (K / 64, rounded up) leaves 5 to 8 steps per wave,
    with the last steps of some waves masked, exact against the oracle: the two-tile MFMA kernel
    (M = 32), the half-tile one (N = 40, 48), and with N = 2064 the whole-tile one."""
    d = synth.w8a8_inputs(M, N, K, seed=7 + K % 97)
    acc_ref, out_ref = w8a8_gemm(d["xq"], d["x_scale"], d["W"], d["w_scale"])
    assert np.array_equal(_run(gpu, d, M, N, K, i32=True), acc_ref)
    assert np.array_equal(_run(gpu, d, M, N, K), out_ref)


@pytest.mark.parametrize("K", [4352, 7232])
@pytest.mark.parametrize("M", [1, 8, 15])
def test_w8a8_dot_kernel_deep_ragged_steps(gpu, monkeypatch, M, K):
    """The VALU dot kernel (forced) at 5 and 8 k-steps per wave, exact against the oracle."""
    monkeypatch.setenv("GQ8_W8A8_KERNEL", "dot")
    N = 40
    d = synth.w8a8_inputs(M, N, K, seed=11 + M)
    acc_ref, _ = w8a8_gemm(d["xq"], d["x_scale"], d["W"], d["w_scale"])
    assert np.array_equal(_run(gpu, d, M, N, K, i32=True), acc_ref)


@pytest.mark.parametrize("M,N,K", [(16, 1536, 4096), (5, 37, 80)])
def test_w8a8_host_pack_equals_device_pack(gpu, M, N, K):
    """gq8_w8a8_pack_host writes the bytes gq8_w8a8_pack writes; the product on them is exact."""
    d = synth.w8a8_inputs(M, N, K, seed=12)
    host = np.zeros(gpu.gq8_w8a8_packed_bytes(K, N), np.int8)
    gpu.gq8_w8a8_pack_host(np.ascontiguousarray(d["W"]), K, N, host)
    dev = _pack(gpu, d["W"])
    torch.cuda.synchronize()
    assert np.array_equal(to_host(dev), host)
    wp = to_dev(host)
    nb = gpu.gq8_workspace_bytes(gpu.OP_W8A8, M, N, K)
    out = torch.empty((M, N), dtype=torch.int16, device="cuda")
    gpu.gq8_w8a8_gemm(to_dev(d["xq"]), to_dev(d["x_scale"]), wp, to_dev(d["w_scale"]), out, M, N, K,
                      workspace(nb), nb)
    torch.cuda.synchronize()
    assert np.array_equal(to_host(out, np.uint16), w8a8_gemm(d["xq"], d["x_scale"], d["W"], d["w_scale"])[1])
