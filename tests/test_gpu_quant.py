"""GPU parity of the weight / activation preparation kernels: Q8_0 and q8_1 quantizers and the
34-byte-block reorder, bit-exact against the oracle (byte work)."""
import numpy as np
import pytest
import torch

from gemm_q8_amd import synth
from gemm_q8_amd.device import q8_0_split_views, to_dev, to_host
from oracle.q8 import quantize_q8_0, quantize_q8_1_bf16

pytestmark = pytest.mark.gpu


def _special_rows():
    w = synth.normal_f32(0, "gpu.q.special", (4, 128), 0.0, 0.02)
    w[0, :32] = 0.0                                           # zero block
    w[0, 32:64] = 1e-9                                        # fp16 scale underflows to 0
    w[1, :32] = 0.0
    w[1, 0] = 127 * 2.0 ** -7
    w[1, 1:5] = np.array([2.5, -2.5, 0.5, 3.5], np.float32) * np.float32(2.0 ** -7)   # ties
    w[2, :32] = 0.0
    w[2, 0] = np.float32(1.49 * 127 * 2.0 ** -24)             # subnormal scale, clamped quants
    w[2, 1] = -w[2, 0]
    return w


@pytest.mark.parametrize("shape", [(4, 128), (37, 96), (1024, 4096)])
def test_q8_0_quantize_bit_exact(gpu, shape):
    w = _special_rows() if shape == (4, 128) else synth.normal_f32(1, "gpu.q.w", shape, 0.0, 0.02)
    rows, K = w.shape
    ref = quantize_q8_0(w)
    buf = torch.empty(gpu.gq8_q8_0_bytes(rows, K), dtype=torch.uint8, device="cuda")
    gpu.gq8_q8_0_quantize(to_dev(w), rows, K, buf)
    torch.cuda.synchronize()
    q, d = q8_0_split_views(buf, rows, K)
    assert np.array_equal(to_host(q).reshape(rows, K // 32, 32), ref.q)
    assert np.array_equal(to_host(d, np.uint16), ref.d)


def test_split_from_blocks_reorders_bytes(gpu):
    rows, K = 9, 160
    ref = quantize_q8_0(synth.normal_f32(2, "gpu.q.b34", (rows, K), 0.0, 0.02))
    b34 = np.zeros((rows, K // 32, 34), np.uint8)
    b34[:, :, 0:2] = ref.d.view(np.uint8).reshape(rows, K // 32, 2)
    b34[:, :, 2:] = ref.q.view(np.uint8)
    buf = torch.empty(gpu.gq8_q8_0_bytes(rows, K), dtype=torch.uint8, device="cuda")
    gpu.gq8_q8_0_split_from_blocks(to_dev(b34), rows, K, buf)
    torch.cuda.synchronize()
    q, d = q8_0_split_views(buf, rows, K)
    assert np.array_equal(to_host(q).reshape(rows, K // 32, 32), ref.q)
    assert np.array_equal(to_host(d, np.uint16), ref.d)


@pytest.mark.parametrize("shape", [(4, 2048), (3, 96)])
def test_q8_1_quantize_bit_exact(gpu, shape):
    x = synth.bf16_normal(3, "gpu.q81", shape)
    rows, K = shape
    ref = quantize_q8_1_bf16(x)
    q = torch.empty((rows, K), dtype=torch.int8, device="cuda")
    d = torch.empty((rows, K // 32), dtype=torch.int16, device="cuda")
    s = torch.empty((rows, K // 32), dtype=torch.int16, device="cuda")
    gpu.gq8_q8_1_quantize(to_dev(x), rows, K, q, d, s)
    torch.cuda.synchronize()
    assert np.array_equal(to_host(q).reshape(ref.q.shape), ref.q)
    assert np.array_equal(to_host(d, np.uint16), ref.d)
    assert np.array_equal(to_host(s, np.uint16), ref.s)
