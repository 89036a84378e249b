"""Hand-worked fixtures under tests/golden/ (each file states its derivation and the passage it
follows): the oracle, the library's host quantizers and its device quantizers must reproduce
them byte for byte."""
import os

import numpy as np
import pytest

from oracle.q8 import quantize_q8_0, quantize_q8_1_bf16

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _load(name):
    out = {}
    for line in open(os.path.join(GOLDEN, name)):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        key, *vals = line.split()
        out[key] = vals
    return out


def _block():
    g = _load("q8_block_inexact_scale.txt")
    w = np.array([np.float32(v) for v in g["q8_0_w"]], np.float32)
    x32 = np.array([np.float32(v) for v in g["q8_1_x"]], np.float32)
    xb = x32.view(np.uint32)
    assert not np.any(xb & 0xFFFF), "every q8_1 input of the fixture is exact in bf16"
    return {
        "w": w[None, :],
        "d0": int(g["q8_0_d"][0], 16),
        "q0": [int(v) for v in g["q8_0_q"]],
        "x": (xb >> 16).astype(np.uint16)[None, :],
        "d1": int(g["q8_1_d"][0], 16),
        "s1": int(g["q8_1_s"][0], 16),
        "q1": [int(v) for v in g["q8_1_q"]],
    }


def test_fixture_is_well_formed():
    b = _block()
    assert b["w"].shape == (1, 32) and b["x"].shape == (1, 32)
    assert len(b["q0"]) == 32 and len(b["q1"]) == 32
    assert sum(b["q1"]) == -119


def test_oracle_reproduces_the_worked_blocks():
    b = _block()
    q0 = quantize_q8_0(b["w"])
    assert int(q0.d[0, 0]) == b["d0"]
    assert q0.q[0, 0].tolist() == b["q0"]
    q1 = quantize_q8_1_bf16(b["x"])
    assert int(q1.d[0, 0]) == b["d1"] and int(q1.s[0, 0]) == b["s1"]
    assert q1.q[0, 0].tolist() == b["q1"]


def test_host_quantizers_reproduce_the_worked_blocks():
    from gemm_q8_amd import gq8
    b = _block()
    buf = np.zeros(gq8.gq8_q8_0_bytes(1, 32), np.uint8)
    gq8.gq8_q8_0_quantize_host(np.ascontiguousarray(b["w"]), 1, 32, buf)
    assert buf[:32].view(np.int8).tolist() == b["q0"]
    assert int(buf[32:34].view(np.uint16)[0]) == b["d0"]
    q = np.zeros(32, np.int8)
    d = np.zeros(1, np.uint16)
    s = np.zeros(1, np.uint16)
    gq8.gq8_q8_1_quantize_host(np.ascontiguousarray(b["x"]), 1, 32, q, d, s)
    assert q.tolist() == b["q1"] and int(d[0]) == b["d1"] and int(s[0]) == b["s1"]


@pytest.mark.gpu
def test_device_quantizers_reproduce_the_worked_blocks(gpu):
    import torch
    from gemm_q8_amd.device import to_dev, to_host
    b = _block()
    buf = torch.zeros(gpu.gq8_q8_0_bytes(1, 32), dtype=torch.uint8, device="cuda")
    gpu.gq8_q8_0_quantize(to_dev(b["w"]), 1, 32, buf)
    q = torch.zeros(32, dtype=torch.int8, device="cuda")
    d = torch.zeros(1, dtype=torch.int16, device="cuda")
    s = torch.zeros(1, dtype=torch.int16, device="cuda")
    gpu.gq8_q8_1_quantize(to_dev(b["x"]), 1, 32, q, d, s)
    torch.cuda.synchronize()
    raw = to_host(buf)
    assert raw[:32].view(np.int8).tolist() == b["q0"]
    assert int(raw[32:34].view(np.uint16)[0]) == b["d0"]
    assert to_host(q).tolist() == b["q1"]
    assert int(to_host(d).view(np.uint16)[0]) == b["d1"]
    assert int(to_host(s).view(np.uint16)[0]) == b["s1"]
