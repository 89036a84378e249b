"""The last-arriver combine (GQ8_COMBINE=last): the down read, the GEMV at T >= 5 and the pair
give bitwise the outputs of the default combine (a kernel of its own), every call leaves the
workspace's arrival counters at zero, repeated calls need no re-zeroing, and a captured graph
replays bitwise with eager work in between."""
import numpy as np
import pytest
import torch

from gemm_q8_amd import synth
from gemm_q8_amd.device import q8_0_from_f32, to_dev, to_host, workspace
from oracle.hc import hc_down
from oracle.q8 import q8_0_gemv, quantize_q8_0
from tests.helpers import check_bf16, check_f32

pytestmark = pytest.mark.gpu


def _down(gpu, wd, R, wn, T, N, K, ws, nb, stream=None, lo=None, rs=None):
    lo = torch.full((T, N), 0x7F7F, dtype=torch.int16, device="cuda") if lo is None else lo
    rs = torch.full((T,), -1.0, dtype=torch.float32, device="cuda") if rs is None else rs
    gpu.gq8_hc_q8_down(wd, R, wn, 1e-6, lo, rs, T, N, K, ws, nb, stream)
    return lo, rs


@pytest.mark.parametrize("T,N,K", [(2, 320, 16384), (4, 320, 16384), (6, 320, 16384), (8, 320, 16384),
                                   (3, 70, 1056), (8, 130, 4128), (5, 64, 96)])
def test_down_last_arriver_is_the_kernel_combine(gpu, monkeypatch, T, N, K):
    d = synth.hc_inputs(T, K=K, N=N, seed=70)
    wd = q8_0_from_f32(to_dev(d["w_down"]))
    R, wn = to_dev(d["R"]), to_dev(d["w_norm"])
    nb = gpu.gq8_workspace_bytes(gpu.OP_HC_DOWN, T, N, K)
    lo0, rs0 = _down(gpu, wd, R, wn, T, N, K, workspace(nb), nb)
    monkeypatch.setenv("GQ8_COMBINE", "last")
    ws = workspace(nb)
    for _ in range(3):                                   # counters left at zero: no re-zeroing
        lo, rs = _down(gpu, wd, R, wn, T, N, K, ws, nb)
        torch.cuda.synchronize()
        assert torch.equal(lo, lo0) and torch.equal(rs, rs0), f"T={T} N={N} K={K}"
        assert gpu.gq8_workspace_check(gpu.OP_HC_DOWN, T, N, K, ws, nb) == 0
    lo_ref, _, S = hc_down(d["R"], d["w_norm"], quantize_q8_0(d["w_down"]))
    check_bf16(to_host(lo, np.uint16), lo_ref, S, f"down last-arriver T={T} N={N} K={K}")


@pytest.mark.parametrize("T,N,K", [(5, 1024, 4096), (8, 1024, 4096), (16, 1024, 4096), (7, 70, 2080),
                                   (12, 33, 8224)])
def test_gemv_last_arriver_is_the_kernel_combine(gpu, monkeypatch, T, N, K):
    w = synth.normal_f32(71, "gpu.comb.w", (N, K), 0.0, 0.02)
    x = synth.normal_f32(71, "gpu.comb.x", (T, K))
    wb, xd = q8_0_from_f32(to_dev(w)), to_dev(x)
    nb = gpu.gq8_workspace_bytes(gpu.OP_Q8_0_GEMV, T, N, K)
    y0 = torch.empty((T, N), dtype=torch.float32, device="cuda")
    gpu.gq8_q8_0_gemv(wb, xd, y0, T, N, K, workspace(nb), nb)
    monkeypatch.setenv("GQ8_COMBINE", "last")
    ws = workspace(nb)
    for _ in range(3):
        y = torch.full_like(y0, 7.0)
        gpu.gq8_q8_0_gemv(wb, xd, y, T, N, K, ws, nb)
        torch.cuda.synchronize()
        assert torch.equal(y, y0), f"T={T} N={N} K={K}"
        assert gpu.gq8_workspace_check(gpu.OP_Q8_0_GEMV, T, N, K, ws, nb) == 0
    y_ref, S = q8_0_gemv(quantize_q8_0(w), x)
    check_f32(to_host(y), y_ref, S, f"gemv last-arriver T={T} N={N} K={K}")


@pytest.mark.parametrize("T", [1, 2, 4, 6])
def test_pair_last_arriver_is_the_default_pair(gpu, monkeypatch, T):
    Nlr, Khc = 320, 16384
    d = synth.hc_inputs(T, seed=72)
    wd, wu = q8_0_from_f32(to_dev(d["w_down"])), q8_0_from_f32(to_dev(d["w_up"]))
    R, wn = to_dev(d["R"]), to_dev(d["w_norm"])
    nb = gpu.gq8_workspace_bytes(gpu.OP_HC_PAIR, T, Nlr, Khc)

    def pair(ws):
        lo = torch.empty((T, Nlr), dtype=torch.int16, device="cuda")
        rs = torch.empty((T,), dtype=torch.float32, device="cuda")
        out = torch.empty((T, Khc), dtype=torch.int16, device="cuda")
        gpu.gq8_hc_q8_pair(wd, R, wn, 1e-6, wu, lo, rs, out, T, Nlr, Khc, ws, nb)
        return lo, rs, out
    ref = pair(workspace(nb))
    monkeypatch.setenv("GQ8_COMBINE", "last")
    ws = workspace(nb)
    for _ in range(2):
        got = pair(ws)
        torch.cuda.synchronize()
        for a, b in zip(got, ref):
            assert torch.equal(a, b), f"T={T}"
        assert gpu.gq8_workspace_check(gpu.OP_HC_PAIR, T, Nlr, Khc, ws, nb) == 0


def test_last_arriver_workspace_reused_for_a_smaller_call(gpu, monkeypatch):
    """One workspace, zeroed once and sized for the larger call, serves a down read at T = 8 and
    then smaller down reads and a GEMV: the counters open the workspace, so each call finds them
    at the same zeroed bytes (the larger call's partial sums lie past them)."""
    big = (8, 320, 16384)
    nb = gpu.gq8_workspace_bytes(gpu.OP_HC_DOWN, *big)
    ws = workspace(nb)
    cases = [("down", big), ("down", (2, 320, 4096)), ("down", (5, 64, 2048)), ("gemv", (6, 1024, 2048))]
    want, got = [], []
    for mode, out in (("kernel", want), ("last", got)):
        monkeypatch.setenv("GQ8_COMBINE", mode)
        for i, (op, (T, N, K)) in enumerate(cases):
            if op == "down":
                d = synth.hc_inputs(T, K=K, N=N, seed=74 + i)
                wd = q8_0_from_f32(to_dev(d["w_down"]))
                lo, rs = _down(gpu, wd, to_dev(d["R"]), to_dev(d["w_norm"]), T, N, K, ws, nb)
                out.append((lo, rs))
            else:
                wg = q8_0_from_f32(to_dev(synth.normal_f32(74, "gpu.comb.r.w", (N, K), 0.0, 0.02)))
                xg = to_dev(synth.normal_f32(74, "gpu.comb.r.x", (T, K)))
                y = torch.full((T, N), 7.0, dtype=torch.float32, device="cuda")
                gpu.gq8_q8_0_gemv(wg, xg, y, T, N, K, ws, nb)
                out.append((y,))
            torch.cuda.synchronize()
    for (op, shape), a, b in zip(cases, want, got):
        for x, y in zip(a, b):
            assert torch.equal(x, y), f"{op} {shape}"
    assert gpu.gq8_workspace_check(gpu.OP_HC_DOWN, *big, ws, nb) == 0


def test_last_arriver_graph_replay(gpu, monkeypatch):
    """The down read and the GEMV (T = 8) with the last-arriver combine captured into one graph and
    replayed five times, with eager work and a poisoned partial-sum region (not the counters)
    between replays: every replay equals the eager result, and the counters are zero after each."""
    monkeypatch.setenv("GQ8_COMBINE", "last")
    T, N, K = 6, 320, 16384
    d = synth.hc_inputs(T, seed=73)
    wd = q8_0_from_f32(to_dev(d["w_down"]))
    R, wn = to_dev(d["R"]), to_dev(d["w_norm"])
    nb = gpu.gq8_workspace_bytes(gpu.OP_HC_DOWN, T, N, K)
    cb = gpu.gq8_workspace_counter_bytes(gpu.OP_HC_DOWN, T, N, K)
    ws = workspace(nb)
    Tg, Ng, Kg = 8, 1024, 4096
    wg = q8_0_from_f32(to_dev(synth.normal_f32(73, "gpu.comb.g.w", (Ng, Kg), 0.0, 0.02)))
    xg = to_dev(synth.normal_f32(73, "gpu.comb.g.x", (Tg, Kg)))
    nbg = gpu.gq8_workspace_bytes(gpu.OP_Q8_0_GEMV, Tg, Ng, Kg)
    wsg = workspace(nbg)
    lo0, rs0 = _down(gpu, wd, R, wn, T, N, K, ws, nb)
    y0 = torch.empty((Tg, Ng), dtype=torch.float32, device="cuda")
    gpu.gq8_q8_0_gemv(wg, xg, y0, Tg, Ng, Kg, wsg, nbg)
    torch.cuda.synchronize()
    lo, rs = torch.empty_like(lo0), torch.empty_like(rs0)
    y = torch.empty_like(y0)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            _down(gpu, wd, R, wn, T, N, K, ws, nb, s, lo, rs)
            gpu.gq8_q8_0_gemv(wg, xg, y, Tg, Ng, Kg, wsg, nbg, s)
    for _ in range(5):
        lo.zero_(); rs.zero_(); y.zero_()
        ws[cb:].fill_(0xFF)                              # partial sums poisoned, counters kept
        torch.cuda.synchronize()
        with torch.cuda.stream(s):
            g.replay()
        torch.cuda.synchronize()
        assert torch.equal(lo, lo0) and torch.equal(rs, rs0) and torch.equal(y, y0)
        assert gpu.gq8_workspace_check(gpu.OP_HC_DOWN, T, N, K, ws, nb) == 0
        assert gpu.gq8_workspace_check(gpu.OP_Q8_0_GEMV, Tg, Ng, Kg, wsg, nbg) == 0
