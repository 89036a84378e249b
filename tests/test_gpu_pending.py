"""The down read and the pair with the pending write (gq8_hc_q8_down_pending,
gq8_hc_q8_pair_pending): R_out is bitwise the oracle's bf16(R + P), and lo, rs and out are bitwise
what the calls without it give on R_out; lo also passes the rules against the oracle's down read
of R_out; a captured graph replays bitwise."""
import numpy as np
import pytest
import torch

from gemm_q8_amd import synth
from gemm_q8_amd.device import q8_0_from_f32, to_dev, to_host, workspace
from oracle.hc import hc_down, pending_write
from oracle.q8 import quantize_q8_0
from tests.helpers import check_bf16

pytestmark = pytest.mark.gpu


def _inputs(T, N, K, seed):
    d = synth.hc_inputs(T, K=K, N=N, seed=seed)
    P = synth.bf16_normal(seed, "gpu.pending.P", (T, K), 0.0, 0.5)
    return d, P


def _t(shape, dtype=torch.int16):
    return torch.full(shape, 0x7F7F if dtype == torch.int16 else -1.0, dtype=dtype, device="cuda")


@pytest.mark.parametrize("T,N,K", [(1, 320, 16384), (4, 320, 16384), (6, 320, 16384),
                                   (9, 320, 16384), (16, 320, 16384), (3, 70, 1056), (12, 33, 544)])
def test_down_pending(gpu, T, N, K):
    d, P = _inputs(T, N, K, 80)
    wd = q8_0_from_f32(to_dev(d["w_down"]))
    R, Pd, wn = to_dev(d["R"]), to_dev(P), to_dev(d["w_norm"])
    nb = gpu.gq8_workspace_bytes(gpu.OP_HC_DOWN, T, N, K)
    ws = workspace(nb)
    Ro, lo, rs = _t((T, K)), _t((T, N)), _t((T,), torch.float32)
    gpu.gq8_hc_q8_down_pending(wd, R, Pd, wn, 1e-6, Ro, lo, rs, T, N, K, ws, nb)
    torch.cuda.synchronize()
    Rp = pending_write(d["R"], P)
    assert np.array_equal(to_host(Ro, np.uint16), Rp), f"R_out T={T} N={N} K={K}"
    lo2, rs2 = _t((T, N)), _t((T,), torch.float32)
    gpu.gq8_hc_q8_down(wd, to_dev(Rp), wn, 1e-6, lo2, rs2, T, N, K, ws, nb)
    torch.cuda.synchronize()
    assert torch.equal(lo, lo2) and torch.equal(rs, rs2)
    lo_ref, rs_ref, S = hc_down(Rp, d["w_norm"], quantize_q8_0(d["w_down"]))
    check_bf16(to_host(lo, np.uint16), lo_ref, S, f"down pending T={T} N={N} K={K}")
    assert np.allclose(to_host(rs), rs_ref, rtol=1e-5, atol=0)


# (1, 64, 1056): the whole-row down read with its fetch-ahead, then the general (LDS-staged) up read
@pytest.mark.parametrize("T,Nlr,Khc", [(1, 320, 16384), (4, 320, 16384), (6, 320, 16384), (2, 64, 1056),
                                       (1, 64, 1056)])
def test_pair_pending(gpu, T, Nlr, Khc):
    d, P = _inputs(T, Nlr, Khc, 81)
    wd, wu = q8_0_from_f32(to_dev(d["w_down"])), q8_0_from_f32(to_dev(d["w_up"]))
    R, Pd, wn = to_dev(d["R"]), to_dev(P), to_dev(d["w_norm"])
    nb = gpu.gq8_workspace_bytes(gpu.OP_HC_PAIR, T, Nlr, Khc)
    ws = workspace(nb)
    Ro, lo, rs, out = _t((T, Khc)), _t((T, Nlr)), _t((T,), torch.float32), _t((T, Khc))
    gpu.gq8_hc_q8_pair_pending(wd, R, Pd, wn, 1e-6, wu, Ro, lo, rs, out, T, Nlr, Khc, ws, nb)
    torch.cuda.synchronize()
    Rp = pending_write(d["R"], P)
    assert np.array_equal(to_host(Ro, np.uint16), Rp)
    lo2, rs2, out2 = _t((T, Nlr)), _t((T,), torch.float32), _t((T, Khc))
    gpu.gq8_hc_q8_pair(wd, to_dev(Rp), wn, 1e-6, wu, lo2, rs2, out2, T, Nlr, Khc, ws, nb)
    torch.cuda.synchronize()
    assert torch.equal(lo, lo2) and torch.equal(rs, rs2) and torch.equal(out, out2)


def test_pair_pending_graph_replay(gpu):
    T, Nlr, Khc = 4, 320, 16384
    d, P = _inputs(T, Nlr, Khc, 82)
    wd, wu = q8_0_from_f32(to_dev(d["w_down"])), q8_0_from_f32(to_dev(d["w_up"]))
    R, Pd, wn = to_dev(d["R"]), to_dev(P), to_dev(d["w_norm"])
    nb = gpu.gq8_workspace_bytes(gpu.OP_HC_PAIR, T, Nlr, Khc)
    ws = workspace(nb)
    bufs = [_t((T, Khc)), _t((T, Nlr)), _t((T,), torch.float32), _t((T, Khc))]
    gpu.gq8_hc_q8_pair_pending(wd, R, Pd, wn, 1e-6, wu, *bufs[:3], bufs[3], T, Nlr, Khc, ws, nb)
    torch.cuda.synchronize()
    ref = [b.clone() for b in bufs]
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            gpu.gq8_hc_q8_pair_pending(wd, R, Pd, wn, 1e-6, wu, *bufs[:3], bufs[3], T, Nlr, Khc,
                                       ws, nb, s)
    cb = gpu.gq8_workspace_counter_bytes(gpu.OP_HC_PAIR, T, Nlr, Khc)
    for _ in range(3):
        for b in bufs:
            b.zero_()
        ws[cb:].fill_(0xFF)
        torch.cuda.synchronize()
        with torch.cuda.stream(s):
            g.replay()
        torch.cuda.synchronize()
        for b, r in zip(bufs, ref):
            assert torch.equal(b, r)
