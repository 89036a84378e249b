"""The allocation-free pair (gq8_hc_q8_pair_noalloc, its workspace a fixed device array inside the
library) against gq8_hc_q8_pair with a caller workspace: bitwise equal lo, rs and out, on two calls
in a row, the second with a smaller input (fewer tokens and a shorter depth), so the second call
reads only what it has itself written to the shared array."""
import numpy as np
import pytest
import torch

from gemm_q8_amd import synth
from gemm_q8_amd.device import q8_0_from_f32, to_dev, workspace

pytestmark = pytest.mark.gpu


def _both(gpu, T, Nlr, Khc, seed):
    d = synth.hc_inputs(T, K=Khc, N=Nlr, seed=seed)
    wd, wu = q8_0_from_f32(to_dev(d["w_down"])), q8_0_from_f32(to_dev(d["w_up"]))
    R, wn = to_dev(d["R"]), to_dev(d["w_norm"])
    res = []
    for noalloc in (False, True):
        lo = torch.full((T, Nlr), 0x5555, dtype=torch.int16, device="cuda")
        rs = torch.full((T,), -1.0, dtype=torch.float32, device="cuda")
        out = torch.full((T, Khc), 0x5555, dtype=torch.int16, device="cuda")
        if noalloc:
            gpu.gq8_hc_q8_pair_noalloc(wd, R, wn, 1e-6, wu, lo, rs, out, T, Nlr, Khc)
        else:
            nb = gpu.gq8_workspace_bytes(gpu.OP_HC_PAIR, T, Nlr, Khc)
            gpu.gq8_hc_q8_pair(wd, R, wn, 1e-6, wu, lo, rs, out, T, Nlr, Khc, workspace(nb), nb)
        res.append((lo, rs, out))
    torch.cuda.synchronize()
    for a, b in zip(*res):
        assert torch.equal(a, b), f"T={T} Nlr={Nlr} Khc={Khc}"


@pytest.mark.parametrize("first,second", [((6, 320, 16384), (1, 320, 16384)),
                                          ((16, 320, 16384), (4, 320, 8192)),
                                          ((5, 96, 4128), (2, 64, 1056))])
def test_noalloc_pair_matches_the_workspace_pair(gpu, first, second):
    _both(gpu, *first, seed=60)
    _both(gpu, *second, seed=61)


@pytest.mark.parametrize("first,second", [((8, 320, 16384), (2, 320, 8192)),
                                          ((4, 1024, 4096), (2, 64, 1056))])
def test_noalloc_pair_last_arriver_after_a_larger_call(gpu, monkeypatch, first, second):
    """With the last-arriver combine the array's arrival counters must be zero before each call:
    they open the array (the same 256 bytes for every pair shape) and every call leaves them at
    zero, so a smaller call after a larger one, whose partial sums cover the bytes that follow,
    still finds them zero."""
    monkeypatch.setenv("GQ8_COMBINE", "last")
    _both(gpu, *first, seed=62)
    _both(gpu, *second, seed=63)


def test_noalloc_pair_limit(gpu):
    """A shape whose workspace exceeds the library's array is refused before any launch."""
    T, Nlr, Khc = 16, 1024, 32768
    assert gpu.gq8_workspace_bytes(gpu.OP_HC_PAIR, T, Nlr, Khc) > gpu.NOALLOC_SCRATCH_BYTES
    st = gpu.raw().gq8_hc_q8_pair_noalloc(1 << 20, 1 << 20, 1 << 20, 1e-6, 1 << 20, 1 << 20, None,
                                          1 << 20, T, Nlr, Khc, None)
    assert st == gpu.ESHAPE
