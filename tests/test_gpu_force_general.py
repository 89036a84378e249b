"""GPU parity of the general kernels at the tuned shapes: with GQ8_FORCE_GENERIC=1 every call
takes the path a shape outside the tuned set would take (the down read then the LDS-staged up
read instead of the fused pair, the work-group GEMV instead of the wave-owned one, the plan-based
routed-expert kernels), checked against the oracle at the full workload sizes; an unknown value is
ignored. Also gq8_workspace_init: it zero-fills, and refuses a capturing stream."""
import numpy as np
import pytest
import torch

from gemm_q8_amd import synth
from gemm_q8_amd.device import q8_0_from_f32, to_dev, to_host, workspace
from oracle.hc import hc_down, hc_up
from oracle.moe import moe_forward, route
from oracle.q8 import q8_0_gemv, quantize_q8_0, quantize_q8_1_bf16
from tests.helpers import check_bf16, check_f32
from tests.test_gpu_moe import _moe_case

pytestmark = pytest.mark.gpu


@pytest.fixture
def forced(monkeypatch):
    monkeypatch.setenv("GQ8_FORCE_GENERIC", "1")


def _pair(gpu, d, T, Nlr=320, Khc=16384):
    wd, wu = q8_0_from_f32(to_dev(d["w_down"])), q8_0_from_f32(to_dev(d["w_up"]))
    nb = gpu.gq8_workspace_bytes(gpu.OP_HC_PAIR, T, Nlr, Khc)
    lo = torch.empty((T, Nlr), dtype=torch.int16, device="cuda")
    rs = torch.empty((T,), dtype=torch.float32, device="cuda")
    out = torch.empty((T, Khc), dtype=torch.int16, device="cuda")
    gpu.gq8_hc_q8_pair(wd, to_dev(d["R"]), to_dev(d["w_norm"]), 1e-6, wu, lo, rs, out, T, Nlr, Khc,
                       workspace(nb), nb)
    torch.cuda.synchronize()
    return to_host(lo, np.uint16), to_host(rs), to_host(out, np.uint16)


@pytest.mark.parametrize("T", [1, 4, 6])
def test_forced_general_pair_full_size(gpu, forced, T):
    d = synth.hc_inputs(T)
    lo, rs, out = _pair(gpu, d, T)
    lo_ref, rs_ref, S = hc_down(d["R"], d["w_norm"], quantize_q8_0(d["w_down"]))
    check_bf16(lo, lo_ref, S, f"forced down T={T}")
    assert np.allclose(rs, rs_ref, rtol=1e-5, atol=0)
    out_ref, S_up = hc_up(lo, quantize_q8_0(d["w_up"]))
    check_bf16(out, out_ref, S_up, f"forced up T={T}")


@pytest.mark.parametrize("T", [1, 2, 3])
def test_forced_general_gemv_full_size(gpu, forced, T):
    d = synth.q8_0_gemv_inputs(T=T)
    nb = gpu.gq8_workspace_bytes(gpu.OP_Q8_0_GEMV, T, 1024, 4096)
    y = torch.empty((T, 1024), dtype=torch.float32, device="cuda")
    gpu.gq8_q8_0_gemv(q8_0_from_f32(to_dev(d["w"])), to_dev(d["x"]), y, T, 1024, 4096, workspace(nb), nb)
    torch.cuda.synchronize()
    y_ref, S = q8_0_gemv(quantize_q8_0(d["w"]), d["x"])
    check_f32(to_host(y), y_ref, S, f"forced gemv T={T}")


@pytest.mark.parametrize("T,E,topk,D,F", [(4, 512, 8, 2048, 512), (3, 20, 4, 128, 256)])
def test_forced_general_moe(gpu, forced, T, E, topk, D, F):
    """The plan-based general kernels at the tuned shapes, on the int8 input (checked against the
    oracle in _moe_case) and on the bf16 input (quantized into the workspace first: bitwise the
    same), and the q8_1(h) option (its down read stays the token kernel) against the oracle."""
    seed = 48
    out, (xq, xd, ids, w, agu, adn, ws, nb) = _moe_case(gpu, T, E, topk, D, F, seed=seed)
    inp = synth.moe_inputs(T=T, E=E, D=D, seed=seed)
    out2 = torch.empty_like(out)
    ws.fill_(0xFF)
    gpu.gq8_moe_q8_0_routed_bf16(to_dev(inp["x"]), ids, w, agu, adn, out2, T, topk, E, D, F, ws, nb)
    o3 = torch.empty_like(out)
    gpu.gq8_moe_q8_0_routed_flags(xq, xd, ids, w, agu, adn, o3, T, topk, E, D, F, gpu.MOE_H_Q8_1, ws, nb)
    torch.cuda.synchronize()
    assert torch.equal(out, out2)
    ids_ref, p_ref = route(inp["logits"], topk)
    experts = lambda e: synth.moe_expert_weights(e, D=D, F=F, seed=seed)  # noqa: E731
    blocks = lambda e: (quantize_q8_0(experts(e)["gate_up"]), quantize_q8_0(experts(e)["down"]))  # noqa: E731
    y_ref, S = moe_forward(quantize_q8_1_bf16(inp["x"]), ids_ref, p_ref, blocks, h_q8_1=True)
    check_bf16(to_host(o3, np.uint16), y_ref, S, f"forced moe q8_1(h) T={T} D={D} F={F}",
               page=False)   # its own rule: h re-quantized on both sides, codes may flip


def test_unknown_switch_value_is_ignored(gpu, monkeypatch):
    T = 1
    d = synth.hc_inputs(T)
    monkeypatch.delenv("GQ8_FORCE_GENERIC", raising=False)
    _, _, ref = _pair(gpu, d, T)
    monkeypatch.setenv("GQ8_FORCE_GENERIC", "yes")
    _, _, out = _pair(gpu, d, T)
    assert np.array_equal(out, ref)                   # the tuned path, bitwise


def test_workspace_init_zero_fills_and_refuses_capture(gpu):
    nb = 4096 + 48
    ws = torch.full((nb,), 0x5A, dtype=torch.uint8, device="cuda")
    gpu.gq8_workspace_init(ws, nb)
    torch.cuda.synchronize()
    assert not ws.any()
    raw = gpu.raw()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            rc = raw.gq8_workspace_init(ws.data_ptr(), nb, s.cuda_stream)
            ws.zero_()                                 # the graph holds one ordinary node
    assert rc == gpu.ECAPTURE


_NOTE_SCRIPT = r"""
import torch
from gemm_q8_amd import gq8
x = torch.zeros((1, 320), dtype=torch.int16, device="cuda")
w = torch.zeros(gq8.gq8_q8_0_bytes(64, 320), dtype=torch.uint8, device="cuda")
out = torch.empty((1, 64), dtype=torch.int16, device="cuda")
for _ in range(3):
    gq8.gq8_hc_q8_up(w, x, out, 1, 64, 320, None, 0)
torch.cuda.synchronize()
print("calls done")
"""


@pytest.mark.parametrize("value,expect", [("1", "gq8: up read: general up kernel"),
                                          ("yes", "gq8: GQ8_FORCE_GENERIC=yes not understood")])
def test_general_path_note_is_said_once(value, expect):
    """A fresh process: three calls, the note on stderr exactly once."""
    import os
    import subprocess
    import sys
    env = dict(os.environ, GQ8_FORCE_GENERIC=value)
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, "-c", _NOTE_SCRIPT], cwd=root, env=env, capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    assert "calls done" in r.stdout
    assert sum(line.startswith(expect) for line in r.stderr.splitlines()) == 1, r.stderr[-2000:]
