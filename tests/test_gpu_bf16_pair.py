"""GPU parity of the BF16 comparison read (the HC down/up pair on BF16 weights) against the
oracle's BF16 reads: lo and rs of the down read, and the up read of the GPU's own lo, at small
ragged shapes and the full 320 x 16384 workload; replay determinism with a poisoned workspace."""
import numpy as np
import pytest
import torch

from gemm_q8_amd import synth
from gemm_q8_amd.device import to_dev, to_host, workspace
from oracle.hc import hc_down_bf16, hc_up_bf16
from tests.helpers import check_bf16

pytestmark = pytest.mark.gpu


def _bf16_pair(gpu, wd, R, wn, wu, T, Nlr, Khc, ws=None):
    nb = gpu.gq8_workspace_bytes(gpu.OP_HC_PAIR, T, Nlr, Khc)
    ws = workspace(nb) if ws is None else ws
    lo = torch.empty((T, Nlr), dtype=torch.int16, device="cuda")
    rs = torch.empty((T,), dtype=torch.float32, device="cuda")
    out = torch.empty((T, Khc), dtype=torch.int16, device="cuda")
    gpu.gq8_hc_bf16_pair(wd, R, wn, 1e-6, wu, lo, rs, out, T, Nlr, Khc, ws, nb)
    return lo, rs, out, ws


@pytest.mark.parametrize("T,Nlr,Khc", [(1, 320, 16384), (4, 320, 16384), (6, 320, 16384),
                                       (16, 320, 2048), (3, 320, 1056), (5, 96, 544),
                                       (2, 64, 4096), (7, 352, 640)])
def test_bf16_pair_matches_oracle(gpu, T, Nlr, Khc):
    d = synth.hc_inputs(T, K=Khc, N=Nlr, seed=50)
    w = synth.hc_weights_bf16(K=Khc, N=Nlr, seed=50)
    lo, rs, out, _ = _bf16_pair(gpu, to_dev(w["w_down"]), to_dev(d["R"]), to_dev(d["w_norm"]),
                                to_dev(w["w_up"]), T, Nlr, Khc)
    torch.cuda.synchronize()
    lo_ref, rs_ref, S = hc_down_bf16(d["R"], d["w_norm"], w["w_down"])
    check_bf16(to_host(lo, np.uint16), lo_ref, S, f"bf16 down T={T} Nlr={Nlr} Khc={Khc}")
    assert np.allclose(to_host(rs), rs_ref, rtol=1e-5, atol=0)
    out_ref, S_up = hc_up_bf16(to_host(lo, np.uint16), w["w_up"])
    check_bf16(to_host(out, np.uint16), out_ref, S_up, f"bf16 up T={T} Nlr={Nlr} Khc={Khc}")


def test_bf16_pair_replay_with_poisoned_workspace(gpu):
    T, Nlr, Khc = 4, 320, 16384
    d = synth.hc_inputs(T, K=Khc, N=Nlr, seed=51)
    w = synth.hc_weights_bf16(K=Khc, N=Nlr, seed=51)
    args = (to_dev(w["w_down"]), to_dev(d["R"]), to_dev(d["w_norm"]), to_dev(w["w_up"]), T, Nlr, Khc)
    lo0, rs0, out0, ws = _bf16_pair(gpu, *args)
    for _ in range(3):
        ws.fill_(0xFF)
        lo, rs, out, _ = _bf16_pair(gpu, *args, ws=ws)
        torch.cuda.synchronize()
        assert torch.equal(lo, lo0) and torch.equal(rs, rs0) and torch.equal(out, out0)


def test_bf16_pair_graph_replay(gpu):
    T, Nlr, Khc = 6, 320, 16384
    d = synth.hc_inputs(T, K=Khc, N=Nlr, seed=52)
    w = synth.hc_weights_bf16(K=Khc, N=Nlr, seed=52)
    wd, R, wn, wu = to_dev(w["w_down"]), to_dev(d["R"]), to_dev(d["w_norm"]), to_dev(w["w_up"])
    lo0, rs0, out0, ws = _bf16_pair(gpu, wd, R, wn, wu, T, Nlr, Khc)
    torch.cuda.synchronize()
    nb = ws.numel()
    lo, rs, out = torch.empty_like(lo0), torch.empty_like(rs0), torch.empty_like(out0)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            gpu.gq8_hc_bf16_pair(wd, R, wn, 1e-6, wu, lo, rs, out, T, Nlr, Khc, ws, nb, s)
    for _ in range(3):
        lo.zero_(); rs.zero_(); out.zero_()
        ws.fill_(0xFF)
        torch.cuda.synchronize()
        with torch.cuda.stream(s):
            g.replay()
        torch.cuda.synchronize()
        assert torch.equal(lo, lo0) and torch.equal(rs, rs0) and torch.equal(out, out0)
