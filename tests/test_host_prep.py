"""CPU parity of the library's host-side preparation (gq8_*_host): the Q8_0 and q8_1 quantizers
and the 34-byte-block reorder, byte-exact against the oracle's quantizers, including zero blocks,
scales that underflow or land in the fp16 subnormals, exact ties, values near the fp16 range
limit, and the argument checks. Also the workspace check (no arrival counters exist)."""
import numpy as np
import pytest

from gemm_q8_amd import synth
from oracle.q8 import quantize_q8_0, quantize_q8_1_bf16


@pytest.fixture(scope="module")
def lib():
    from gemm_q8_amd import gq8
    return gq8


def _special_rows():
    w = synth.normal_f32(5, "host.q.special", (6, 128), 0.0, 0.02)
    w[0, :32] = 0.0                                           # zero block
    w[0, 32:64] = 1e-9                                        # fp16 scale underflows to 0
    w[1, :32] = 0.0
    w[1, 0] = 127 * 2.0 ** -7
    w[1, 1:5] = np.array([2.5, -2.5, 0.5, 3.5], np.float32) * np.float32(2.0 ** -7)   # ties
    w[2, :32] = 0.0
    w[2, 0] = np.float32(1.49 * 127 * 2.0 ** -24)             # subnormal scale, clamped quants
    w[2, 1] = -w[2, 0]
    w[3, :32] = np.linspace(-8.0e6, 8.0e6, 32, dtype=np.float32)   # scale near the fp16 maximum
    w[4, :32] = np.float32(3.0e-6) * np.arange(-16, 16, dtype=np.float32)   # subnormal scales
    w[5, 32:64] = -0.0
    return w


def _split(rows, K, buf):
    q = buf[: rows * K].view(np.int8).reshape(rows, K // 32, 32)
    d = buf[rows * K:].view(np.uint16).reshape(rows, K // 32)
    return q, d


@pytest.mark.parametrize("shape", [None, (37, 96), (64, 4096)])
def test_q8_0_quantize_host_matches_oracle(lib, shape):
    w = _special_rows() if shape is None else synth.normal_f32(6, "host.q.w", shape, 0.0, 0.02)
    rows, K = w.shape
    ref = quantize_q8_0(w)
    buf = np.full(lib.gq8_q8_0_bytes(rows, K), 0xAB, np.uint8)
    lib.gq8_q8_0_quantize_host(np.ascontiguousarray(w), rows, K, buf)
    q, d = _split(rows, K, buf)
    assert np.array_equal(q, ref.q)
    assert np.array_equal(d, ref.d)


def test_split_from_blocks_host_reorders_bytes(lib):
    rows, K = 9, 160
    ref = quantize_q8_0(synth.normal_f32(7, "host.q.b34", (rows, K), 0.0, 0.02))
    b34 = np.zeros((rows, K // 32, 34), np.uint8)
    b34[:, :, 0:2] = ref.d.view(np.uint8).reshape(rows, K // 32, 2)
    b34[:, :, 2:] = ref.q.view(np.uint8)
    buf = np.zeros(lib.gq8_q8_0_bytes(rows, K), np.uint8)
    lib.gq8_q8_0_split_from_blocks_host(b34, rows, K, buf)
    q, d = _split(rows, K, buf)
    assert np.array_equal(q, ref.q)
    assert np.array_equal(d, ref.d)


@pytest.mark.parametrize("shape", [(4, 2048), (3, 96)])
def test_q8_1_quantize_host_matches_oracle(lib, shape):
    rows, K = shape
    x = synth.bf16_normal(8, "host.q81", shape)
    x[0, :32] = 0                                             # a zero block
    x[-1, :32] = 0x3F80                                       # 1.0 everywhere: q = 127, s = 32 * 127 * d
    ref = quantize_q8_1_bf16(x)
    q = np.zeros((rows, K), np.int8)
    d = np.zeros((rows, K // 32), np.uint16)
    s = np.zeros((rows, K // 32), np.uint16)
    lib.gq8_q8_1_quantize_host(x, rows, K, q, d, s)
    assert np.array_equal(q.reshape(ref.q.shape), ref.q)
    assert np.array_equal(d, ref.d)
    assert np.array_equal(s, ref.s)
    q2 = np.zeros((rows, K), np.int8)
    lib.gq8_q8_1_quantize_host(x, rows, K, q2, d, None)       # the sum field is optional
    assert np.array_equal(q2, q)


def test_host_prep_argument_checks(lib):
    raw = lib.raw()
    dummy = 1 << 20  # never dereferenced: every case fails validation first
    assert raw.gq8_q8_0_quantize_host(dummy, 4, 48, dummy) == lib.ESHAPE
    assert raw.gq8_q8_0_quantize_host(dummy, -1, 64, dummy) == lib.EINVAL
    assert raw.gq8_q8_0_quantize_host(None, 4, 64, dummy) == lib.EINVAL
    assert raw.gq8_q8_0_quantize_host(None, 0, 64, None) == lib.OK
    assert raw.gq8_q8_0_split_from_blocks_host(dummy, 4, 40, dummy) == lib.ESHAPE
    assert raw.gq8_q8_0_split_from_blocks_host(dummy, 4, 64, None) == lib.EINVAL
    assert raw.gq8_q8_1_quantize_host(dummy, 2, 33, dummy, dummy, None) == lib.ESHAPE
    assert raw.gq8_q8_1_quantize_host(dummy, 2, 64, dummy, None, None) == lib.EINVAL


def test_workspace_check_without_counters(lib):
    # operations without arrival counters: nothing to read, 0
    assert lib.gq8_workspace_check(lib.OP_W8A8, 16, 1536, 4096, None, 0) == 0
    assert lib.gq8_workspace_check(lib.OP_HC_UP, 4, 16384, 320, None, 0) == 0
    buf = np.zeros(256, np.uint8)
    # the binding refuses host arrays and CPU tensors where device memory is required, and GPU
    # memory where host memory is required, before calling the library
    with pytest.raises(ValueError):
        lib.gq8_workspace_check(lib.OP_HC_DOWN, 1, 320, 16384, buf, buf.nbytes)
    # a workspace smaller than the operation's: refused before any read
    raw = lib.raw()
    st = raw.gq8_workspace_check(lib.OP_HC_DOWN, 1, 320, 16384, 1 << 20, 16, None, buf.ctypes.data)
    assert st == lib.EWORKSPACE
    import torch
    with pytest.raises(ValueError):
        lib.gq8_q8_0_gemv(torch.zeros(64, dtype=torch.uint8), None, None, 1, 1, 32, None, 0, 0)
    with pytest.raises(ValueError):
        lib.gq8_q8_1_quantize_host(np.zeros((4, 64), np.uint16)[:, :32], 4, 32,
                                   np.zeros(128, np.int8), np.zeros(4, np.uint16))
    raw = lib.raw()
    assert raw.gq8_workspace_check(lib.OP_HC_DOWN, 1, 320, 16384, None, 64, None, None) == lib.EINVAL


@pytest.mark.parametrize("K,N", [(4096, 48), (80, 17), (16, 1)])
def test_w8a8_pack_host_places_every_byte(lib, K, N):
    """Every W[k][n] lands in slot (n // 16, k // 64, 16 (k % 64 // 16) + n % 16) at byte k % 16, and
    the padding past K or N is zero."""
    W = synth.int8_uniform(9, "host.w8.pack", (K, N))
    nb = lib.gq8_w8a8_packed_bytes(K, N)
    buf = np.full(nb, 0x55, np.int8)
    lib.gq8_w8a8_pack_host(np.ascontiguousarray(W), K, N, buf)
    ksteps = (K + 63) // 64
    slots = buf.reshape((N + 15) // 16, ksteps, 64, 16)
    k = np.arange(K)[:, None]
    n = np.arange(N)[None, :]
    got = slots[n // 16, k // 64, 16 * ((k % 64) // 16) + n % 16, k % 16]
    assert np.array_equal(got, W)
    mask = np.zeros(slots.shape, bool)
    mask[n // 16, k // 64, 16 * ((k % 64) // 16) + n % 16, k % 16] = True
    assert not slots[~mask].any()
    raw = lib.raw()
    assert raw.gq8_w8a8_pack_host(1 << 20, 40, 8, 1 << 20) == lib.ESHAPE
    assert raw.gq8_w8a8_pack_host(None, 64, 8, 1 << 20) == lib.EINVAL
