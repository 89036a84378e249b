"""GPU parity of the Q8_0 reads against the oracle: the Q8_0 matrix-vector product (T = 1..16),
the fused RMSNorm + Q8_0 down read and the up read, at small ragged shapes and at the full
workload sizes, plus exactness, determinism, graph-replay and workspace invariants."""
import numpy as np
import pytest
import torch

from gemm_q8_amd import synth
from gemm_q8_amd.device import q8_0_from_f32, to_dev, to_host, workspace
from oracle.hc import hc_down, hc_up
from oracle.numerics import bf16_to_f32, fp16_to_f32
from oracle.q8 import q8_0_gemv, quantize_q8_0
from tests.helpers import check_bf16, check_f32

pytestmark = pytest.mark.gpu


def _gemv(gpu, wbuf, x, T, N, K):
    nb = gpu.gq8_workspace_bytes(gpu.OP_Q8_0_GEMV, T, N, K)
    ws = workspace(nb)
    y = torch.empty((T, N), dtype=torch.float32, device="cuda")
    gpu.gq8_q8_0_gemv(wbuf, x, y, T, N, K, ws, nb)
    return y, ws, nb


@pytest.mark.parametrize("T,N,K", [(1, 96, 4096), (3, 37, 1056), (5, 130, 2080), (8, 64, 96),
                                   (11, 33, 320), (16, 70, 4096), (2, 5, 32), (4, 300, 1024),
                                   (2, 77, 3104), (3, 9, 2080), (1, 1, 64), (2, 1, 4096),
                                   (1, 333, 4064), (3, 130, 4096),
                                   # 256-column slabs from T = 5: slab counts off a multiple of 8
                                   # (general work-group mapping), a 32- or 64-column last slab
                                   (6, 64, 288), (12, 70, 2080), (9, 129, 4160), (16, 16, 8224)])
def test_gemv_matches_oracle(gpu, T, N, K):
    w = synth.normal_f32(10, "gpu.gemv.w", (N, K), 0.0, 0.02)
    x = synth.normal_f32(10, "gpu.gemv.x", (T, K))
    y, _, _ = _gemv(gpu, q8_0_from_f32(to_dev(w)), to_dev(x), T, N, K)
    y_ref, S = q8_0_gemv(quantize_q8_0(w), x)
    check_f32(to_host(y), y_ref, S, f"gemv T={T} N={N} K={K}")


@pytest.mark.parametrize("T", [1, 2, 4, 8, 16])
def test_gemv_full_size(gpu, T):
    d = synth.q8_0_gemv_inputs(T=T)
    y, _, _ = _gemv(gpu, q8_0_from_f32(to_dev(d["w"])), to_dev(d["x"]), T, 1024, 4096)
    y_ref, S = q8_0_gemv(quantize_q8_0(d["w"]), d["x"])
    check_f32(to_host(y), y_ref, S, f"gemv full T={T}")


def test_gemv_one_hot_is_exact(gpu):
    N, K = 50, 2048
    w = synth.normal_f32(11, "gpu.gemv.oh", (N, K), 0.0, 0.02)
    ks = [0, 31, 32, 1023, 1024, 2047]
    x = np.zeros((len(ks), K), np.float32)
    for t, k in enumerate(ks):
        x[t, k] = 1.0
    b = quantize_q8_0(w)
    y, _, _ = _gemv(gpu, q8_0_from_f32(to_dev(w)), to_dev(x), len(ks), N, K)
    y = to_host(y)
    for t, k in enumerate(ks):
        want = fp16_to_f32(b.d[:, k // 32]) * b.q[:, k // 32, k % 32].astype(np.float32)
        assert np.array_equal(y[t], want)


@pytest.mark.parametrize("N,K", [(31, 4096), (7, 2080)])
def test_gemv_one_hot_few_rows_is_exact(gpu, N, K):
    """The wave-owned kernel (T <= 3): one-hot x gives d * q exactly (all other terms are zeros)."""
    w = synth.normal_f32(12, "gpu.gemv.oh3", (N, K), 0.0, 0.02)
    ks = [0, 1023, K - 1]
    b = quantize_q8_0(w)
    for T in (1, 2, 3):
        x = np.zeros((T, K), np.float32)
        for t in range(T):
            x[t, ks[t]] = 1.0
        y, _, _ = _gemv(gpu, q8_0_from_f32(to_dev(w)), to_dev(x), T, N, K)
        y = to_host(y)
        for t in range(T):
            k = ks[t]
            want = fp16_to_f32(b.d[:, k // 32]) * b.q[:, k // 32, k % 32].astype(np.float32)
            assert np.array_equal(y[t], want), f"T={T} k={k}"


def test_gemv_reads_the_scales(gpu):
    """Perturbing one block scale changes exactly that row's outputs (the Q8_0 bytes are read)."""
    N, K, T = 40, 1024, 2
    w = synth.normal_f32(12, "gpu.gemv.sc", (N, K), 0.0, 0.02)
    x = to_dev(synth.normal_f32(12, "gpu.gemv.scx", (T, K)))
    wbuf = q8_0_from_f32(to_dev(w))
    y0, _, _ = _gemv(gpu, wbuf, x, T, N, K)
    sc = wbuf[N * K:].view(torch.float16)
    sc[7 * (K // 32) + 3] *= 2
    y1, _, _ = _gemv(gpu, wbuf, x, T, N, K)
    diff = (to_host(y0) != to_host(y1)).any(axis=0)
    assert diff.tolist() == [n == 7 for n in range(N)]


def test_gemv_repeat_calls_bitwise(gpu):
    T, N, K = 4, 1024, 4096
    d = synth.q8_0_gemv_inputs(T=T)
    wbuf, x = q8_0_from_f32(to_dev(d["w"])), to_dev(d["x"])
    y0, _, _ = _gemv(gpu, wbuf, x, T, N, K)
    for _ in range(3):
        y1, _, _ = _gemv(gpu, wbuf, x, T, N, K)
        torch.cuda.synchronize()
        assert torch.equal(y0, y1)


@pytest.mark.parametrize("T", [1, 6])
def test_down_workspace_poison_and_replay(gpu, T):
    """Every call rewrites every partial sum it reads: poisoning the workspace between calls
    (NaN bit patterns) changes nothing, and a captured graph replays bitwise (T = 1: the
    whole-row kernel, which does not touch the workspace)."""
    N, K = 320, 16384
    d = synth.hc_inputs(T)
    wd = q8_0_from_f32(to_dev(d["w_down"]))
    R, wn = to_dev(d["R"]), to_dev(d["w_norm"])
    nb = gpu.gq8_workspace_bytes(gpu.OP_HC_DOWN, T, N, K)
    ws = workspace(nb)
    lo0 = torch.empty((T, N), dtype=torch.int16, device="cuda")
    rs0 = torch.empty((T,), dtype=torch.float32, device="cuda")
    gpu.gq8_hc_q8_down(wd, R, wn, 1e-6, lo0, rs0, T, N, K, ws, nb)
    torch.cuda.synchronize()
    lo, rs = torch.zeros_like(lo0), torch.zeros_like(rs0)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            gpu.gq8_hc_q8_down(wd, R, wn, 1e-6, lo, rs, T, N, K, ws, nb, s)
    for _ in range(3):
        ws.fill_(0xFF)
        lo.zero_()
        rs.zero_()
        torch.cuda.synchronize()
        with torch.cuda.stream(s):
            g.replay()
        torch.cuda.synchronize()
        assert torch.equal(lo, lo0) and torch.equal(rs, rs0)


def test_gemv_graph_replay_bitwise(gpu):
    T, N, K = 6, 512, 4096
    w = synth.normal_f32(13, "gpu.gemv.g", (N, K), 0.0, 0.02)
    x = to_dev(synth.normal_f32(13, "gpu.gemv.gx", (T, K)))
    wbuf = q8_0_from_f32(to_dev(w))
    y_direct, ws, nb = _gemv(gpu, wbuf, x, T, N, K)
    torch.cuda.synchronize()
    y = torch.zeros_like(y_direct)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            gpu.gq8_q8_0_gemv(wbuf, x, y, T, N, K, ws, nb, s)
    for _ in range(3):
        y.zero_()
        torch.cuda.synchronize()
        with torch.cuda.stream(s):
            g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y_direct)


def test_gemv_empty_and_zero_k(gpu):
    y = torch.full((2, 8), 7.0, device="cuda")
    gpu.gq8_q8_0_gemv(None, None, y, 2, 8, 0, None, 0)
    torch.cuda.synchronize()
    assert int(y.count_nonzero()) == 0
    gpu.gq8_q8_0_gemv(None, None, None, 0, 8, 64, None, 0)   # T = 0: nothing to do


# ------------------------------------------------------------------------------ hyper-connection

def _down(gpu, wbuf, R, wn, T, N, K, eps=1e-6):
    nb = gpu.gq8_workspace_bytes(gpu.OP_HC_DOWN, T, N, K)
    ws = workspace(nb)
    lo = torch.empty((T, N), dtype=torch.int16, device="cuda")
    rs = torch.empty((T,), dtype=torch.float32, device="cuda")
    gpu.gq8_hc_q8_down(wbuf, R, wn, eps, lo, rs, T, N, K, ws, nb)
    return lo, rs


def _up(gpu, wbuf, lo, T, N, K):
    nb = gpu.gq8_workspace_bytes(gpu.OP_HC_UP, T, N, K)
    ws = workspace(nb)
    out = torch.empty((T, N), dtype=torch.int16, device="cuda")
    gpu.gq8_hc_q8_up(wbuf, lo, out, T, N, K, ws, nb)
    return out


@pytest.mark.parametrize("T,N,K", [(1, 37, 2048), (4, 10, 1056), (6, 64, 96), (16, 9, 4096),
                                   (8, 70, 1536), (9, 33, 544),
                                   # from T = 9 two waves per tile, one per 256-column half: a
                                   # 32-column last slab (its second half empty), ragged row groups
                                   (12, 70, 1056), (16, 130, 2112)])
def test_down_matches_oracle_small(gpu, T, N, K):
    d = synth.hc_inputs(T, K=K, N=N, seed=20)
    lo, rs = _down(gpu, q8_0_from_f32(to_dev(d["w_down"])), to_dev(d["R"]), to_dev(d["w_norm"]), T, N, K)
    lo_ref, rs_ref, S = hc_down(d["R"], d["w_norm"], quantize_q8_0(d["w_down"]))
    check_bf16(to_host(lo, np.uint16), lo_ref, S, f"down T={T} N={N} K={K}")
    assert np.allclose(to_host(rs), rs_ref, rtol=1e-5, atol=0)


@pytest.mark.parametrize("N,K", [(1, 32), (37, 96), (65, 1056), (320, 16384), (9, 20512), (130, 33792)])
def test_down_whole_rows(gpu, N, K):
    """T = 1 runs the whole-row down kernel (a work-group owns two rows and all of K, 1024-column
    chunks per wave): an odd row count (the last work-group's second row clamped), K below one
    chunk, a chunk cut short (K % 1024 != 0), and more than sixteen chunks (waves taking a second
    and third chunk), against the oracle; repeated calls are bitwise equal."""
    T = 1
    d = synth.hc_inputs(T, K=K, N=N, seed=21)
    wd, R, wn = q8_0_from_f32(to_dev(d["w_down"])), to_dev(d["R"]), to_dev(d["w_norm"])
    lo, rs = _down(gpu, wd, R, wn, T, N, K)
    lo2, rs2 = _down(gpu, wd, R, wn, T, N, K)
    torch.cuda.synchronize()
    assert torch.equal(lo, lo2) and torch.equal(rs, rs2)
    lo_ref, rs_ref, S = hc_down(d["R"], d["w_norm"], quantize_q8_0(d["w_down"]))
    check_bf16(to_host(lo, np.uint16), lo_ref, S, f"down rows N={N} K={K}")
    assert np.allclose(to_host(rs), rs_ref, rtol=1e-5, atol=0)


@pytest.mark.parametrize("T", [1, 4, 6])
def test_hc_pair_full_size(gpu, T):
    d = synth.hc_inputs(T)
    bd, bu = quantize_q8_0(d["w_down"]), quantize_q8_0(d["w_up"])
    wd, wu = q8_0_from_f32(to_dev(d["w_down"])), q8_0_from_f32(to_dev(d["w_up"]))
    lo, rs = _down(gpu, wd, to_dev(d["R"]), to_dev(d["w_norm"]), T, 320, 16384)
    lo_ref, rs_ref, S = hc_down(d["R"], d["w_norm"], bd)
    lo_h = to_host(lo, np.uint16)
    check_bf16(lo_h, lo_ref, S, f"down full T={T}")
    assert np.allclose(to_host(rs), rs_ref, rtol=1e-5, atol=0)

    # up read on its own: the same bf16 input on both sides (the oracle's own rounding of lo)
    from oracle.numerics import bf16_bits
    lo_in = bf16_bits(lo_ref.astype(np.float32))
    out = _up(gpu, wu, to_dev(lo_in), T, 16384, 320)
    out_ref, S_up = hc_up(lo_in, bu)
    check_bf16(to_host(out, np.uint16), out_ref, S_up, f"up full T={T}")

    # chained: GPU down -> GPU up against oracle down -> oracle up, tolerance widened by the
    # bf16 rounding of lo (one spacing either way) and the down read's own tolerance
    out2 = _up(gpu, wu, lo, T, 16384, 320)
    ref_chain, _ = hc_up(lo_in, bu)
    from oracle.q8 import dequantize
    from oracle.numerics import bf16_ulp
    Wu = np.abs(dequantize(bu))
    dlo = 2e-3 * S + bf16_ulp(np.abs(lo_ref) + 2e-3 * S)
    S_chain = S_up + dlo @ Wu.T / 2e-3
    check_bf16(to_host(out2, np.uint16), ref_chain, S_chain, f"hc chain T={T}",
               page=False)   # lo differs by bf16 roundings on the two sides: widened rule above


@pytest.mark.parametrize("T,N,K", [(1, 100, 320), (4, 77, 320), (6, 5, 64), (9, 40, 1024), (16, 33, 320),
                                   (2, 50, 640), (7, 70, 960), (3, 21, 352)])
def test_up_matches_oracle_small(gpu, T, N, K):
    w = synth.normal_f32(21, "gpu.up.w", (N, K), 0.0, 0.02)
    lo = synth.bf16_normal(21, "gpu.up.lo", (T, K))
    out = _up(gpu, q8_0_from_f32(to_dev(w)), to_dev(lo), T, N, K)
    ref, S = hc_up(lo, quantize_q8_0(w))
    check_bf16(to_host(out, np.uint16), ref, S, f"up T={T} N={N} K={K}")


def test_down_scale_invariance_on_gpu(gpu):
    """R scaled by 4 leaves lo unchanged up to rounding: rs is applied after the dot."""
    T, N, K = 2, 64, 4096
    d = synth.hc_inputs(T, K=K, N=N, seed=22)
    wd = q8_0_from_f32(to_dev(d["w_down"]))
    R4 = (bf16_to_f32(d["R"]) * np.float32(4.0)).view(np.uint32) >> np.uint32(16)
    lo1, rs1 = _down(gpu, wd, to_dev(d["R"]), to_dev(d["w_norm"]), T, N, K)
    lo4, rs4 = _down(gpu, wd, to_dev(R4.astype(np.uint16)), to_dev(d["w_norm"]), T, N, K)
    a = bf16_to_f32(to_host(lo1, np.uint16))
    b = bf16_to_f32(to_host(lo4, np.uint16))
    assert np.allclose(a, b, rtol=2 ** -7, atol=1e-6)
    assert np.allclose(to_host(rs1), 4 * to_host(rs4), rtol=1e-5)


def _pair(gpu, wd, R, wn, wu, T, Nlr, Khc, ws=None, stream=None, lo=None, rs=None, out=None):
    nb = gpu.gq8_workspace_bytes(gpu.OP_HC_PAIR, T, Nlr, Khc)
    ws = workspace(nb) if ws is None else ws
    lo = torch.empty((T, Nlr), dtype=torch.int16, device="cuda") if lo is None else lo
    rs = torch.empty((T,), dtype=torch.float32, device="cuda") if rs is None else rs
    out = torch.empty((T, Khc), dtype=torch.int16, device="cuda") if out is None else out
    gpu.gq8_hc_q8_pair(wd, R, wn, 1e-6, wu, lo, rs, out, T, Nlr, Khc, ws, nb, stream)
    return lo, rs, out


# T = 1 at depths 1056, 544 and 32: up reads of 16.5, 8.5 and 0.5 work-groups of 64 rows, so the
# down launch's fetch-ahead work-groups cover a partial last one
@pytest.mark.parametrize("T,Nlr,Khc", [(1, 320, 16384), (4, 320, 16384), (6, 320, 16384),
                                       (16, 320, 16384), (3, 320, 1056), (8, 64, 2048),
                                       (5, 96, 544), (1, 320, 1056), (1, 320, 544), (1, 320, 32)])
def test_pair_is_the_two_calls(gpu, T, Nlr, Khc):
    """The pair entry (two kernels for Nlr = 320, the combine inside the up read) gives bitwise the
    down call's lo and rs and the up call's output on that lo."""
    d = synth.hc_inputs(T, K=Khc, N=Nlr, seed=40)
    wd, wu = q8_0_from_f32(to_dev(d["w_down"])), q8_0_from_f32(to_dev(d["w_up"]))
    R, wn = to_dev(d["R"]), to_dev(d["w_norm"])
    lo_p, rs_p, out_p = _pair(gpu, wd, R, wn, wu, T, Nlr, Khc)
    lo_s, rs_s = _down(gpu, wd, R, wn, T, Nlr, Khc)
    out_s = _up(gpu, wu, lo_s, T, Khc, Nlr)
    torch.cuda.synchronize()
    assert torch.equal(lo_p, lo_s)
    assert torch.equal(rs_p, rs_s)
    assert torch.equal(out_p, out_s)
    # and the pair's up output against the oracle's up read of the pair's own lo
    out_ref, S_up = hc_up(to_host(lo_p, np.uint16), quantize_q8_0(d["w_up"]))
    check_bf16(to_host(out_p, np.uint16), out_ref, S_up, f"pair up T={T} Nlr={Nlr} Khc={Khc}")


def _tiled(gpu, w_split, rows, K):
    wt = torch.empty_like(w_split)
    gpu.gq8_q8_0_tile16(w_split, rows, K, 1, wt)
    return wt


@pytest.mark.parametrize("T,N,K", [(1, 16384, 320), (6, 16384, 320), (16, 48, 960), (3, 64, 640)])
def test_up_tiled_is_the_split_read(gpu, T, N, K):
    """gq8_hc_q8_up_tiled on the weights tiled by gq8_q8_0_tile16: bitwise the split-layout up
    read."""
    d = synth.hc_inputs(T, K=N, N=K, seed=42)          # up weight [N][K] = the pair's w_up
    wu = q8_0_from_f32(to_dev(d["w_up"]))
    lo = to_dev(synth.bf16_normal(42, "gpu.up.tiled.lo", (T, K), 0.0, 1.0))
    out_s = _up(gpu, wu, lo, T, N, K)
    out_t = torch.full_like(out_s, 0x5555)
    gpu.gq8_hc_q8_up_tiled(_tiled(gpu, wu, N, K), lo, out_t, T, N, K, None, 0)
    torch.cuda.synchronize()
    assert torch.equal(out_t, out_s), f"T={T} N={N} K={K}"


@pytest.mark.parametrize("T,Nlr,Khc", [(1, 320, 16384), (2, 320, 16384), (4, 320, 16384),
                                       (6, 320, 16384), (16, 320, 16384), (3, 640, 2048)])
def test_pair_tiled_is_the_pair(gpu, T, Nlr, Khc):
    """gq8_hc_q8_pair_tiled (up weights tiled): lo, rs and out bitwise those of gq8_hc_q8_pair,
    on every path (whole-row down read at T = 1, the up kernel with the combine for T <= 4,
    three kernels above, and an up depth of 640)."""
    d = synth.hc_inputs(T, K=Khc, N=Nlr, seed=43)
    wd, wu = q8_0_from_f32(to_dev(d["w_down"])), q8_0_from_f32(to_dev(d["w_up"]))
    R, wn = to_dev(d["R"]), to_dev(d["w_norm"])
    lo_s, rs_s, out_s = _pair(gpu, wd, R, wn, wu, T, Nlr, Khc)
    nb = gpu.gq8_workspace_bytes(gpu.OP_HC_PAIR, T, Nlr, Khc)
    lo_t = torch.full_like(lo_s, 0x5555)
    rs_t = torch.full_like(rs_s, -1.0)
    out_t = torch.full_like(out_s, 0x5555)
    gpu.gq8_hc_q8_pair_tiled(wd, R, wn, 1e-6, _tiled(gpu, wu, Khc, Nlr), lo_t, rs_t, out_t, T, Nlr,
                             Khc, workspace(nb), nb)
    torch.cuda.synchronize()
    assert torch.equal(lo_t, lo_s) and torch.equal(rs_t, rs_s) and torch.equal(out_t, out_s), f"T={T}"


def test_pair_graph_replay_and_poison(gpu):
    T, Nlr, Khc = 6, 320, 16384
    d = synth.hc_inputs(T, seed=41)
    wd, wu = q8_0_from_f32(to_dev(d["w_down"])), q8_0_from_f32(to_dev(d["w_up"]))
    R, wn = to_dev(d["R"]), to_dev(d["w_norm"])
    nb = gpu.gq8_workspace_bytes(gpu.OP_HC_PAIR, T, Nlr, Khc)
    ws = workspace(nb)
    lo0, rs0, out0 = _pair(gpu, wd, R, wn, wu, T, Nlr, Khc, ws=ws)
    torch.cuda.synchronize()
    lo, rs = torch.empty_like(lo0), torch.empty_like(rs0)
    out = torch.empty_like(out0)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            _pair(gpu, wd, R, wn, wu, T, Nlr, Khc, ws=ws, stream=s, lo=lo, rs=rs, out=out)
    for _ in range(3):
        lo.zero_(); rs.zero_(); out.zero_()
        ws.fill_(0x7F)                     # partial planes and sums of squares poisoned
        torch.cuda.synchronize()
        with torch.cuda.stream(s):
            g.replay()
        torch.cuda.synchronize()
        assert torch.equal(lo, lo0) and torch.equal(rs, rs0) and torch.equal(out, out0)


@pytest.mark.parametrize("T", [1, 3, 8])
def test_gemv_long_rows(gpu, T):
    """K = 20480: more 1 KiB chunks than the 16 waves of a work-group (VALU path), 40 slabs (MFMA)."""
    N, K = 48, 20480
    w = synth.normal_f32(12, "gpu.gemv.long.w", (N, K), 0.0, 0.02)
    x = synth.normal_f32(12, "gpu.gemv.long.x", (T, K))
    y, _, _ = _gemv(gpu, q8_0_from_f32(to_dev(w)), to_dev(x), T, N, K)
    torch.cuda.synchronize()
    y_ref, S = q8_0_gemv(quantize_q8_0(w), x)
    check_f32(to_host(y), y_ref, S, f"gemv long T={T}")


@pytest.mark.parametrize("T,Nlr,Khc", [(2, 1024, 4096), (5, 1024, 2080)])
def test_pair_widest_low_rank(gpu, T, Nlr, Khc):
    """Nlr = 1024, the widest up depth (four 320-column chunks, the last ragged)."""
    d = synth.hc_inputs(T, K=Khc, N=Nlr, seed=42)
    wd, wu = q8_0_from_f32(to_dev(d["w_down"])), q8_0_from_f32(to_dev(d["w_up"]))
    lo, rs, out = _pair(gpu, wd, to_dev(d["R"]), to_dev(d["w_norm"]), wu, T, Nlr, Khc)
    torch.cuda.synchronize()
    lo_ref, rs_ref, S = hc_down(d["R"], d["w_norm"], quantize_q8_0(d["w_down"]))
    check_bf16(to_host(lo, np.uint16), lo_ref, S, f"pair down T={T} Nlr={Nlr}")
    assert np.allclose(to_host(rs), rs_ref, rtol=1e-5, atol=0)
    out_ref, S_up = hc_up(to_host(lo, np.uint16), quantize_q8_0(d["w_up"]))
    check_bf16(to_host(out, np.uint16), out_ref, S_up, f"pair up T={T} Nlr={Nlr}")


def test_gemv_mfma_graph_replay(gpu):
    """The T >= 5 GEMV (slab partials in the workspace, then the combine) in a hipGraph: replays
    with the workspace poisoned in between equal the eager result."""
    T, N, K = 8, 1024, 4096
    w = synth.normal_f32(13, "gpu.gemv.g.w", (N, K), 0.0, 0.02)
    x = to_dev(synth.normal_f32(13, "gpu.gemv.g.x", (T, K)))
    wb = q8_0_from_f32(to_dev(w))
    y0, ws, nb = _gemv(gpu, wb, x, T, N, K)
    torch.cuda.synchronize()
    y = torch.empty_like(y0)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            gpu.gq8_q8_0_gemv(wb, x, y, T, N, K, ws, nb, s)
    for _ in range(3):
        y.zero_()
        ws.fill_(0xFF)
        torch.cuda.synchronize()
        with torch.cuda.stream(s):
            g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y0)


# ------------------------------------------------------------------------------ exact, full size

def _one_hot_cols(T, K, stride_mix):
    """T distinct columns spread over K (different blocks and slabs for each token)."""
    return [int((t * K // T + stride_mix * (t + 1) + 37 * t) % K) for t in range(T)]


_CS = [1.0, -1.5, 0.75, -3.0]


@pytest.mark.parametrize("general", [False, True])
@pytest.mark.parametrize("T", [1, 4, 6, 16])
def test_up_one_hot_full_size_is_exact(gpu, T, general, monkeypatch):
    """lo[t] = c_t e_{k_t} at the full 16384 x 320 up read: every output is one product
    d q c (11 + 7 + 2 significant bits: exact in fp32) and the other 319 terms are exact zeros, so
    out[t] = bf16(d q c) bit for bit, on the direct kernel and on the general (LDS-staged) one. A
    dropped or misread Q8_0 block shows as a wrong row. Values are compared, so a quant of 0 with
    c < 0 may come out as +0 (the sum of the 320 terms) where the single product is -0."""
    from oracle.numerics import bf16_bits
    N, K = 16384, 320
    w = synth.normal_f32(30, "gpu.up.onehot", (N, K), 0.0, 0.02)
    b = quantize_q8_0(w)
    ks = _one_hot_cols(T, K, 7)
    lo = np.zeros((T, K), np.uint16)
    for t, k in enumerate(ks):
        lo[t, k] = bf16_bits(np.float32(_CS[t % 4]))
    if general:
        monkeypatch.setenv("GQ8_FORCE_GENERIC", "1")
    out = to_host(_up(gpu, q8_0_from_f32(to_dev(w)), to_dev(lo), T, N, K), np.uint16)
    for t, k in enumerate(ks):
        prod = (fp16_to_f32(b.d[:, k // 32]) * b.q[:, k // 32, k % 32].astype(np.float32)
                * np.float32(_CS[t % 4])).astype(np.float32)
        assert np.array_equal(bf16_to_f32(out[t]), bf16_to_f32(bf16_bits(prod))), f"T={T} t={t} k={k}"


def _down_one_hot_ref(b, ks, cs, K, eps=1e-6):
    """lo[t][n] = rs_t c_t d[n][k_t/32] q[n][k_t] and rs_t = 1/sqrt(c_t^2 / K + eps) (fp64)."""
    rs = np.array([1.0 / np.sqrt(c * c / K + eps) for c in cs])
    lo = np.stack([rs[t] * cs[t] * fp16_to_f32(b.d[:, k // 32]).astype(np.float64)
                   * b.q[:, k // 32, k % 32].astype(np.float64) for t, k in enumerate(ks)])
    return lo, rs


def _one_hot_R(T, K, ks, cs):
    from oracle.numerics import bf16_bits
    R = np.zeros((T, K), np.uint16)
    for t, k in enumerate(ks):
        R[t, k] = bf16_bits(np.float32(cs[t]))
    return R


@pytest.mark.parametrize("T", [1, 4, 6, 16])
def test_down_one_hot_full_size(gpu, T):
    """R[t] = c_t e_{k_t}, w_norm = 1, at the full 320 x 16384 down read: each lo is one product
    rs c d q, so lo is within one bf16 spacing of the fp64 value for all 320 rows (rs is an fp32
    value on the GPU), and rs within fp32 rounding. The k_t fall in different 512-column slabs; a
    dropped or misread block gives a wrong (or zero) row."""
    N, K = 320, 16384
    w = synth.normal_f32(31, "gpu.down.onehot", (N, K), 0.0, 0.02)
    b = quantize_q8_0(w)
    ks = _one_hot_cols(T, K, 515)
    cs = [_CS[t % 4] for t in range(T)]
    wn = np.full(K, 0x3F80, np.uint16)                           # bf16 1.0
    lo, rs = _down(gpu, q8_0_from_f32(to_dev(w)), to_dev(_one_hot_R(T, K, ks, cs)), to_dev(wn), T, N, K)
    lo_ref, rs_ref = _down_one_hot_ref(b, ks, cs, K)
    from oracle.numerics import bf16_ulp
    v = bf16_to_f32(to_host(lo, np.uint16)).astype(np.float64)
    assert np.all(np.abs(v - lo_ref) <= bf16_ulp(lo_ref)), f"T={T} ks={ks}"
    assert np.allclose(to_host(rs), rs_ref, rtol=2e-7, atol=0)


@pytest.mark.parametrize("T", [1, 4, 6, 16])
def test_pair_one_hot_full_size(gpu, T):
    """The pair (the down's combine inside the up kernel for T <= 4, three kernels above) on the
    one-hot R of the test above: lo within one bf16 spacing of rs c d q, and the up output against
    the oracle's up read of the pair's own lo under both rules."""
    Nlr, Khc = 320, 16384
    wd_f = synth.normal_f32(32, "gpu.pair.onehot.d", (Nlr, Khc), 0.0, 0.02)
    wu_f = synth.normal_f32(32, "gpu.pair.onehot.u", (Khc, Nlr), 0.0, 0.02)
    ks = _one_hot_cols(T, Khc, 301)
    cs = [_CS[(t + 1) % 4] for t in range(T)]
    wn = np.full(Khc, 0x3F80, np.uint16)
    lo, rs, out = _pair(gpu, q8_0_from_f32(to_dev(wd_f)), to_dev(_one_hot_R(T, Khc, ks, cs)),
                        to_dev(wn), q8_0_from_f32(to_dev(wu_f)), T, Nlr, Khc)
    torch.cuda.synchronize()
    lo_ref, rs_ref = _down_one_hot_ref(quantize_q8_0(wd_f), ks, cs, Khc)
    from oracle.numerics import bf16_ulp
    lo_h = to_host(lo, np.uint16)
    v = bf16_to_f32(lo_h).astype(np.float64)
    assert np.all(np.abs(v - lo_ref) <= bf16_ulp(lo_ref)), f"T={T} ks={ks}"
    assert np.allclose(to_host(rs), rs_ref, rtol=2e-7, atol=0)
    out_ref, S_up = hc_up(lo_h, quantize_q8_0(wu_f))
    check_bf16(to_host(out, np.uint16), out_ref, S_up, f"pair one-hot up T={T}")
