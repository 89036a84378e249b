#!/usr/bin/env python3
"""Benchmark of the decode-time Q8_0 read on one MI355X.

Workload (one "step"): the fused RMSNorm + Q8_0 hyper-connection down read (W_down Q8_0
[320, 16384], R bf16 [T, 16384]) followed by the Q8_0 up read (W_up Q8_0 [16384, 320]) on its
output, one gq8_hc_q8_pair call for each T in {1, 4, 6}: 3 x 11,141,120 weight bytes. Every pair reads its
own copy of the weights; the copies rotate through a working set larger than twice the
Infinity Cache (MALL) plus the L2s, so the weight bytes come from HBM. Inputs are seeded and
synthetic (gemm_q8_amd.synth), resident in HBM before the timed region. Calls are captured
serially on one stream into hipGraphs and replayed.

Output: one JSON line on stdout (metric = weight bytes / time in GB/s), with
  roofline      the pair call's algorithmic bytes / its average duration (HIP events on the
                launch stream, graphs of back-to-back calls), against 8 TB/s; the call is two
                kernels (the down read's partial sums, then the up read with the down's
                combine inside), whose separate durations the rocprofv3 summary gives;
  config        per-T pair call times: the mean, the median and p90 over --reps samples of one
                rotation each, and a hot-cache run (one weight set: cache, not HBM, context only);
                the sha256 of the library that ran;
  configs       one record per workload shape of the five configurations (Q8_0 GEMV
                1024 x 4096 at T = 1, 2, 4, 8, 16; the HC pair at T = 1, 4, 6; W8A8 M = 16,
                N = 1536, K = 4096; W8A8 M in {1, 4, 8, 16, 32} x (2560, 4096), (4096, 2048); the
                routed MoE): median / p90 / mean us per call over samples of back-to-back graph
                replays on rotated weight copies, weight GB/s, the fraction of 8 TB/s and of a
                same-byte read probe timed the same way, and the oracle's host time (one BLAS
                thread and the whole pool; a stated sample where the whole call would be slow);
  cpu_baseline  the CPU oracle timed on a bounded sample of the step's workload, at one thread and
                at the whole BLAS pool (host CPU model and thread counts stated).
--all-configs also times comparison reads and variants (BF16 pair, W8A8 on a bf16 x, MoE options,
the read-probe curve) and writes their lines to --report (default bench_all.jsonl) and stderr;
--only, --w8a8-ms and --gemv-ts select among them.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0
WS_TARGET = 640 << 20          # working set per rotation: > 2 x (256 MB MALL + 8 x 4 MB L2)
TS = (1, 4, 6)
K_HC, N_LR = 16384, 320
# the HC-Q8 page's kernel-level times on an Arc Pro B70 (us per down+up read, Q8_0), for context
PAGE_US = {1: 24.7, 4: 29.3, 6: 34.4}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ------------------------------------------------------------------------------------ helpers

class GraphSteps:
    """Captures steps (each a list of launch callables) into hipGraphs on `stream` and replays
    them on that same stream so that exactly K steps run: replays of a full-rotation graph plus
    one remainder graph, all captured before any timed region (prepare)."""

    def __init__(self, torch, stream, step_fns, steps_per_graph):
        self.torch, self.stream = torch, stream
        self.step_fns = step_fns
        self.steps_per_graph = steps_per_graph
        self.g_full = self._capture(steps_per_graph)
        self.rem = {}

    def _capture(self, n):
        torch = self.torch
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(self.stream):
            for i in range(n):                      # eager pass first (lazy init outside capture)
                for f in self.step_fns(i):
                    f(self.stream)
            self.stream.synchronize()
            with torch.cuda.graph(g, stream=self.stream):
                for i in range(n):
                    for f in self.step_fns(i):
                        f(self.stream)
        self.stream.synchronize()
        return g

    def prepare(self, K):
        r = K % self.steps_per_graph
        if r and r not in self.rem:
            self.rem[r] = self._capture(r)
        return self

    def run(self, K):
        full, r = divmod(K, self.steps_per_graph)
        assert r == 0 or r in self.rem, "prepare(K) before run(K)"
        with self.torch.cuda.stream(self.stream):   # replay() launches on the current stream
            for _ in range(full):
                self.g_full.replay()
            if r:
                self.rem[r].replay()


def time_region(torch, stream, fn):
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    fn()
    e1.record(stream)
    e1.synchronize()
    return e0.elapsed_time(e1) * 1e-3       # seconds


def timed_dist(torch, stream, fn_for_set, n_sets, reps=30, min_calls=400):
    """Per-call microseconds of fn_for_set(i) (i = 0 .. n_sets-1 rotates over the weight copies)
    captured serially into one hipGraph: one warm-up rotation, then `reps` samples, each of enough
    whole rotations for >= min_calls calls (so the graph launch itself is amortized). Returns the
    median, p90 and mean over the samples."""
    rot = max(1, -(-min_calls // n_sets))
    gs = GraphSteps(torch, stream, lambda step: [fn_for_set(step)], n_sets)
    gs.run(n_sets)
    us = np.array([time_region(torch, stream, lambda: gs.run(n_sets * rot)) / (n_sets * rot) * 1e6
                   for _ in range(reps)])
    return {"median": float(np.median(us)), "p90": float(np.percentile(us, 90)),
            "mean": float(np.mean(us)), "calls_per_sample": n_sets * rot, "samples": reps}


def code_digest(root, files):
    """sha256 of the sources' code: comments and whitespace removed, so that a change to the
    comments alone keeps the digest and any change to the code changes it."""
    import hashlib
    import re
    h = hashlib.sha256()
    for f in files:
        text = open(os.path.join(root, f)).read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()


def recorded_traffic(per_t=False):
    """HBM bytes per pair call from the committed FETCH_SIZE / WRITE_SIZE summary (per T with
    per_t), or None when the kernel code has changed since those counters were taken."""
    root = os.path.dirname(os.path.abspath(__file__))
    path = os.path.join(root, "profiles", "hc_pair_traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    ok = code_digest(root, rec["sources"]) == rec["kernel_code_sha256"]
    if not ok:
        return None
    return rec.get("per_T_bytes") if per_t else rec["traffic_bytes_per_pair_call"]


def n_sets_for(nbytes, multiple=1):
    n = int(np.ceil(WS_TARGET / nbytes))
    return int(np.ceil(n / multiple) * multiple)


# ------------------------------------------------------------------------------------ HC workload

def setup_hc(torch, gq8, synth, dev):
    from gemm_q8_amd.device import q8_0_from_f32, to_dev, workspace
    base = synth.hc_inputs(6)
    wd0 = q8_0_from_f32(to_dev(base["w_down"]))
    wu0 = q8_0_from_f32(to_dev(base["w_up"]))
    pair_bytes = wd0.numel() + wu0.numel()
    n_sets = n_sets_for(pair_bytes, len(TS))
    wds = [wd0] + [wd0.clone() for _ in range(n_sets - 1)]
    wus = [wu0] + [wu0.clone() for _ in range(n_sets - 1)]
    per_t = {}
    for T in TS:
        d = synth.hc_inputs(T)
        nbd = gq8.gq8_workspace_bytes(gq8.OP_HC_PAIR, T, N_LR, K_HC)
        nbu = gq8.gq8_workspace_bytes(gq8.OP_HC_UP, T, K_HC, N_LR)
        per_t[T] = dict(
            R=to_dev(d["R"]), wn=to_dev(d["w_norm"]),
            lo=torch.empty((T, N_LR), dtype=torch.int16, device=dev),
            rs=torch.empty((T,), dtype=torch.float32, device=dev),
            out=torch.empty((T, K_HC), dtype=torch.int16, device=dev),
            wsd=workspace(nbd), nbd=nbd, wsu=workspace(nbu), nbu=nbu)
    return dict(wds=wds, wus=wus, n_sets=n_sets, per_t=per_t, pair_bytes=pair_bytes)


def hc_down_fn(gq8, h, T, i):
    p = h["per_t"][T]
    w = h["wds"][i % h["n_sets"]]
    return lambda s: gq8.gq8_hc_q8_down(w, p["R"], p["wn"], 1e-6, p["lo"], p["rs"], T, N_LR, K_HC,
                                        p["wsd"], p["nbd"], s)


def hc_up_fn(gq8, h, T, i):
    p = h["per_t"][T]
    w = h["wus"][i % h["n_sets"]]
    return lambda s: gq8.gq8_hc_q8_up(w, p["lo"], p["out"], T, K_HC, N_LR, p["wsu"], p["nbu"], s)


def hc_pair_fn(gq8, h, T, i):
    p = h["per_t"][T]
    wd = h["wds"][i % h["n_sets"]]
    wu = h["wus"][i % h["n_sets"]]
    return lambda s: gq8.gq8_hc_q8_pair(wd, p["R"], p["wn"], 1e-6, wu, p["lo"], p["rs"], p["out"],
                                        T, N_LR, K_HC, p["wsd"], p["nbd"], s)


def hc_pair_tiled_fn(gq8, h, wus_t, T, i):
    """The pair call with the up weights in the tiled layout (gq8_q8_0_tile16 copies of h's)."""
    p = h["per_t"][T]
    wd = h["wds"][i % h["n_sets"]]
    wu = wus_t[i % h["n_sets"]]
    return lambda s: gq8.gq8_hc_q8_pair_tiled(wd, p["R"], p["wn"], 1e-6, wu, p["lo"], p["rs"],
                                              p["out"], T, N_LR, K_HC, p["wsd"], p["nbd"], s)


def hc_step_fns(gq8, h):
    def fns(step):
        return [hc_pair_fn(gq8, h, T, step * len(TS) + j) for j, T in enumerate(TS)]
    return fns


def hc_kernel_bytes(kind, T):
    """Algorithmic bytes of one call: weights + activations read + outputs written."""
    w = K_HC * N_LR + K_HC * N_LR // 32 * 2
    down = w + T * K_HC * 2 + K_HC * 2 + T * N_LR * 2 + T * 4
    up = w + T * N_LR * 2 + T * K_HC * 2
    return {"down": down, "up": up, "pair": down + up}[kind]


# ------------------------------------------------------------------------------------ CPU baseline

def lib_sha256(path):
    import hashlib
    return hashlib.sha256(open(path, "rb").read()).hexdigest()


def cpu_model():
    """The host CPU as /proc/cpuinfo names it: model name, then family / model / stepping."""
    f = {}
    try:
        for line in open("/proc/cpuinfo"):
            k, _, v = line.partition(":")
            k = k.strip()
            if k in ("model name", "cpu family", "model", "stepping") and k not in f:
                f[k] = v.strip()
            if len(f) == 4:
                break
    except OSError:
        return "unknown"
    return (f"{f.get('model name', 'unknown')} (family {f.get('cpu family', '?')}, model "
            f"{f.get('model', '?')}, stepping {f.get('stepping', '?')})")


def cpu_baseline(synth, budget_s):
    """The C++ oracle (test infrastructure: float64 loops, OpenMP over output rows) on the step's
    workload, down + up read at full size for T = 1, 4, 6 per step, repeated for about a third of
    `budget_s` on one thread and two thirds on every host core."""
    from oracle import c_oracle as C
    from oracle.q8 import quantize_q8_0
    base = synth.hc_inputs(6)
    bd, bu = quantize_q8_0(base["w_down"]), quantize_q8_0(base["w_up"])
    ins = {T: synth.hc_inputs(T) for T in TS}
    cores = C.threads_available()

    def run(budget, threads):
        steps, t0 = 0, time.perf_counter()
        while True:
            for T in TS:
                lo, _, _ = C.hc_down(ins[T]["R"], ins[T]["w_norm"], bd, threads=threads)
                C.hc_up(C.bf16_bits(lo.astype(np.float32)), bu, threads=threads)
            steps += 1
            el = time.perf_counter() - t0
            if el >= budget:
                return steps, el
    step_bytes = len(TS) * 2 * (K_HC * N_LR + K_HC * N_LR // 32 * 2)
    run(0.2, 0)                                                    # warm-up
    s1, e1 = run(budget_s / 3, 1)
    sa, ea = run(budget_s * 2 / 3, 0)
    return {"value": round(sa * step_bytes / ea / 1e9, 4), "unit": "GB/s", "cores": int(cores),
            "kind": "oracle", "value_1thread": round(s1 * step_bytes / e1 / 1e9, 4),
            "cpu_model": cpu_model(), "host_threads": os.cpu_count(),
            "sample": f"C++ oracle (float64 loops, OpenMP over output rows): {sa} steps (down+up read "
                      f"at T=1,4,6 each, full size) in {ea:.1f} s on {cores} threads, {s1} steps in "
                      f"{e1:.1f} s on 1 thread"}


# ------------------------------------------------------------------------------------ other configs

def bench_other_configs(torch, gq8, synth, dev, stream, report, only=None, w8a8_ms=None, gemv_ts=None,
                        samples=None):
    from gemm_q8_amd.device import q8_0_from_f32, to_dev, workspace
    lines = []
    only = set(only or ("probe", "combine", "hcbf16", "gemv", "w8a8", "w8a8kern", "moe"))
    ms = tuple(w8a8_ms or (1, 4, 8, 16, 32))

    def emit(d):
        lines.append(d)
        log(json.dumps(d))

    def timed(fn_for_set, n_sets, reps=30):
        # the per-configuration records' method: median over samples of >= 400 calls each
        return timed_dist(torch, stream, fn_for_set, n_sets, reps=samples or max(5, reps // 5))["median"]

    # read-bandwidth probe at the same byte counts
    # (4 KiB: one work-group, the launch floor; the large sizes: how close a plain stream gets)
    for nbytes in (4096, 4_456_448, 5_570_560, 6_291_456, 8_388_608, 10_485_760, 33_554_432,
                   134_217_728, 536_870_912) if "probe" in only else ():
        n = min(n_sets_for(nbytes), 256)         # the 4 KiB floor needs no rotation
        bufs = [torch.ones(nbytes, dtype=torch.uint8, device=dev) for _ in range(n)]
        sink = torch.empty(gq8.gq8_read_probe_sink_floats(nbytes), dtype=torch.float32, device=dev)
        us = timed(lambda i: (lambda s, b=bufs[i % n]: gq8.gq8_read_probe(b, nbytes, sink, s)), n)
        emit({"workload": "read probe", "bytes": nbytes, "us_per_call": round(us, 3),
              "GBps": round(nbytes / us / 1e3, 1)})
        del bufs

    if "combine" in only:
        bench_combine(torch, gq8, synth, dev, stream, emit)
    if "hcbf16" in only:
        bench_hc_bf16(torch, gq8, synth, dev, timed, emit)
    if "gemv" in only:
        bench_gemv_sweep(torch, gq8, synth, dev, timed, emit, gemv_ts)
    if "w8a8" in only:
        bench_w8a8_sweep(torch, gq8, synth, dev, timed, emit, ms)
    if "w8a8kern" in only:
        bench_w8a8_kernels(torch, gq8, synth, dev, timed, emit)
    if "moe" in only:
        bench_moe(torch, gq8, synth, dev, timed, emit)
    if report:
        os.makedirs(os.path.dirname(report) or ".", exist_ok=True)
        with open(report, "w") as f:
            for d in lines:
                f.write(json.dumps(d) + "\n")


def bench_combine(torch, gq8, synth, dev, stream, emit, rounds=3):
    """The split reads' two combines in the same run: a kernel of its own (the default) against
    the last-arriving work-group of each row group (GQ8_COMBINE=last), alternating, for the GEMV
    at T = 5, 8, 16 (1024 x 4096), the down read at T = 1, 4, 8 and the pair at T = 1, 4
    (320 x 16384). Median us per call over graphs of back-to-back calls on rotated weights."""
    from gemm_q8_amd.device import q8_0_from_f32, to_dev, workspace
    h = setup_hc(torch, gq8, synth, dev)
    d = synth.q8_0_gemv_inputs(T=16)
    w0 = q8_0_from_f32(to_dev(d["w"]))
    ng = n_sets_for(w0.numel())
    wg = [w0] + [w0.clone() for _ in range(ng - 1)]
    cases = []
    for T in (5, 8, 16):
        x = to_dev(np.ascontiguousarray(d["x"][:T]))
        y = torch.empty((T, 1024), dtype=torch.float32, device=dev)
        nb = gq8.gq8_workspace_bytes(gq8.OP_Q8_0_GEMV, T, 1024, 4096)
        wsp = workspace(nb)
        cases.append((f"Q8_0 GEMV 1024x4096 T={T}", ng, lambda i, T=T, x=x, y=y, nb=nb, wsp=wsp: (
            lambda s, w=wg[i % ng]: gq8.gq8_q8_0_gemv(w, x, y, T, 1024, 4096, wsp, nb, s))))
    for T in (1, 4, 8):
        dd = synth.hc_inputs(T)
        R, wn = to_dev(dd["R"]), to_dev(dd["w_norm"])
        lo = torch.empty((T, N_LR), dtype=torch.int16, device=dev)
        rs = torch.empty((T,), dtype=torch.float32, device=dev)
        nb = gq8.gq8_workspace_bytes(gq8.OP_HC_DOWN, T, N_LR, K_HC)
        wsp = workspace(nb)
        cases.append((f"HC down read 320x16384 T={T}", h["n_sets"], lambda i, T=T, R=R, wn=wn, lo=lo, rs=rs, nb=nb, wsp=wsp: (
            lambda s, w=h["wds"][i % h["n_sets"]]: gq8.gq8_hc_q8_down(w, R, wn, 1e-6, lo, rs, T, N_LR, K_HC, wsp, nb, s))))
    for T in (1, 4):
        cases.append((f"HC pair T={T}", h["n_sets"], lambda i, T=T: hc_pair_fn(gq8, h, T, i)))
    for name, n, mk in cases:
        t = {"kernel": [], "last": []}
        for _ in range(rounds):
            for mode in ("kernel", "last"):
                os.environ["GQ8_COMBINE"] = mode
                t[mode].append(timed_dist(torch, stream, mk, n, reps=10)["median"])
        os.environ.pop("GQ8_COMBINE", None)
        emit({"workload": "combine of split partial sums: " + name,
              "kernel_combine_us": round(min(t["kernel"]), 3), "last_arriver_us": round(min(t["last"]), 3),
              "rounds": rounds})
    del wg


def bench_hc_bf16(torch, gq8, synth, dev, timed, emit):
    """The BF16 comparison read: the HC pair on BF16 weights against the Q8_0 pair, same harness
    (per-call graphs over rotated weight copies), T in {1, 4, 6}."""
    from gemm_q8_amd.device import q8_0_from_f32, to_dev, workspace
    wb = synth.hc_weights_bf16()
    bd0, bu0 = to_dev(wb["w_down"]), to_dev(wb["w_up"])
    base = synth.hc_inputs(1)
    qd0, qu0 = q8_0_from_f32(to_dev(base["w_down"])), q8_0_from_f32(to_dev(base["w_up"]))
    bf_bytes = (bd0.numel() + bu0.numel()) * 2
    q8_bytes = qd0.numel() + qu0.numel()
    nb_, nq = n_sets_for(bf_bytes), n_sets_for(q8_bytes)
    bds = [bd0] + [bd0.clone() for _ in range(nb_ - 1)]
    bus = [bu0] + [bu0.clone() for _ in range(nb_ - 1)]
    qds = [qd0] + [qd0.clone() for _ in range(nq - 1)]
    qus = [qu0] + [qu0.clone() for _ in range(nq - 1)]
    for T in TS:
        d = synth.hc_inputs(T)
        R, wn = to_dev(d["R"]), to_dev(d["w_norm"])
        lo = torch.empty((T, N_LR), dtype=torch.int16, device=dev)
        rs = torch.empty((T,), dtype=torch.float32, device=dev)
        out = torch.empty((T, K_HC), dtype=torch.int16, device=dev)
        nbw = gq8.gq8_workspace_bytes(gq8.OP_HC_PAIR, T, N_LR, K_HC)
        wsp = workspace(nbw)
        us_b = timed(lambda i: (lambda s, a=bds[i % nb_], b=bus[i % nb_]: gq8.gq8_hc_bf16_pair(
            a, R, wn, 1e-6, b, lo, rs, out, T, N_LR, K_HC, wsp, nbw, s)), nb_)
        us_q = timed(lambda i: (lambda s, a=qds[i % nq], b=qus[i % nq]: gq8.gq8_hc_q8_pair(
            a, R, wn, 1e-6, b, lo, rs, out, T, N_LR, K_HC, wsp, nbw, s)), nq)
        emit({"workload": "HC pair on BF16 weights (comparison read) 320x16384 + 16384x320", "T": T,
              "us_per_call": round(us_b, 3), "weight_GBps": round(bf_bytes / us_b / 1e3, 1),
              "q8_0_pair_us": round(us_q, 3), "bf16_over_q8_0": round(us_b / us_q, 3)})
    del bds, bus, qds, qus


def bench_gemv_sweep(torch, gq8, synth, dev, timed, emit, gemv_ts=None):
    from gemm_q8_amd.device import q8_0_from_f32, to_dev, workspace
    # Q8_0 GEMV N=1024 K=4096, T sweep
    d = synth.q8_0_gemv_inputs(T=16)
    w0 = q8_0_from_f32(to_dev(d["w"]))
    n = n_sets_for(w0.numel())
    ws_ = [w0] + [w0.clone() for _ in range(n - 1)]
    for T in tuple(gemv_ts or (1, 2, 4, 8, 16)):
        x = to_dev(np.ascontiguousarray(d["x"][:T]))
        y = torch.empty((T, 1024), dtype=torch.float32, device=dev)
        nb = gq8.gq8_workspace_bytes(gq8.OP_Q8_0_GEMV, T, 1024, 4096)
        wsp = workspace(nb)
        us = timed(lambda i, T=T, x=x, y=y, nb=nb, wsp=wsp: (
            lambda s, w=ws_[i % n]: gq8.gq8_q8_0_gemv(w, x, y, T, 1024, 4096, wsp, nb, s)), n)
        emit({"workload": "Q8_0 GEMV N=1024 K=4096", "T": T, "us_per_call": round(us, 3),
              "weight_GBps": round(w0.numel() / us / 1e3, 1)})
    del ws_


def bench_w8a8_sweep(torch, gq8, synth, dev, timed, emit, ms):
    from gemm_q8_amd.device import to_dev, workspace
    # W8A8: the M = 16 product, then the sweep over M
    for (M, N, K) in [(16, 1536, 4096)] * (16 in ms) + [(m, 2560, 4096) for m in ms] + \
                     [(m, 4096, 2048) for m in ms]:
        dd = synth.w8a8_inputs(M, N, K)
        wp0 = torch.empty(gq8.gq8_w8a8_packed_bytes(K, N), dtype=torch.int8, device=dev)
        gq8.gq8_w8a8_pack(to_dev(dd["W"]), K, N, wp0)
        n = n_sets_for(wp0.numel())
        wps = [wp0] + [wp0.clone() for _ in range(n - 1)]
        xq, xs, wsc = to_dev(dd["xq"]), to_dev(dd["x_scale"]), to_dev(dd["w_scale"])
        out = torch.empty((M, N), dtype=torch.int16, device=dev)
        nb = gq8.gq8_workspace_bytes(gq8.OP_W8A8, M, N, K)
        wsp = workspace(nb)
        us = timed(lambda i: (lambda s, w=wps[i % n]: gq8.gq8_w8a8_gemm(xq, xs, w, wsc, out, M, N, K, wsp, nb, s)), n)
        emit({"workload": "W8A8", "M": M, "N": N, "K": K, "us_per_call": round(us, 3),
              "weight_GBps": round(N * K / us / 1e3, 1)})
        # the same product on a bf16 x: per-token quantization inside the product kernel, against
        # the quantize kernel followed by the int8 product
        db = synth.w8a8_bf16_inputs(M, N, K)
        xb = to_dev(db["x"])
        xq2 = torch.empty((M, K), dtype=torch.int8, device=dev)
        xs2 = torch.empty((M,), dtype=torch.float32, device=dev)
        nbx = gq8.gq8_workspace_bytes(gq8.OP_W8A8_BF16X, M, N, K)
        wsx = workspace(nbx)
        us = timed(lambda i: (lambda s, w=wps[i % n]: gq8.gq8_w8a8_gemm_bf16x(
            xb, w, wsc, out, None, None, M, N, K, wsx, nbx, s)), n)
        emit({"workload": "W8A8 on a bf16 x" + (" (per-token quantization fused)" if nbx == 0 else
                                                " (two kernels, staged in the workspace)"),
              "M": M, "N": N, "K": K, "us_per_call": round(us, 3), "weight_GBps": round(N * K / us / 1e3, 1)})

        def two(s, w):
            gq8.gq8_quantize_per_token(xb, M, K, xq2, xs2, s)
            gq8.gq8_w8a8_gemm(xq2, xs2, w, wsc, out, M, N, K, wsp, nb, s)
        us = timed(lambda i: (lambda s, w=wps[i % n]: two(s, w)), n)
        emit({"workload": "W8A8 on a bf16 x (quantize kernel, then the product)", "M": M, "N": N,
              "K": K, "us_per_call": round(us, 3), "weight_GBps": round(N * K / us / 1e3, 1)})
        del wps


def bench_w8a8_kernels(torch, gq8, synth, dev, timed, emit, ms=(1, 2, 4, 8)):
    """The VALU dot4 kernel against the int8 MFMA kernel (the default) at the M where both exist,
    each forced with GQ8_W8A8_KERNEL (read by the library on every call, so at graph capture),
    the same inputs and rotated weight copies."""
    from gemm_q8_amd.device import to_dev, workspace
    for (N, K) in ((1536, 4096), (2560, 4096), (4096, 2048)):
        for M in ms:
            dd = synth.w8a8_inputs(M, N, K)
            wp0 = torch.empty(gq8.gq8_w8a8_packed_bytes(K, N), dtype=torch.int8, device=dev)
            gq8.gq8_w8a8_pack(to_dev(dd["W"]), K, N, wp0)
            n = n_sets_for(wp0.numel())
            wps = [wp0] + [wp0.clone() for _ in range(n - 1)]
            xq, xs, wsc = to_dev(dd["xq"]), to_dev(dd["x_scale"]), to_dev(dd["w_scale"])
            out = torch.empty((M, N), dtype=torch.int16, device=dev)
            nb = gq8.gq8_workspace_bytes(gq8.OP_W8A8, M, N, K)
            wsp = workspace(nb)
            rec = {"workload": "W8A8 kernel choice: VALU dot4 against int8 MFMA", "M": M, "N": N, "K": K,
                   "default": "mfma"}
            prev = os.environ.get("GQ8_W8A8_KERNEL")
            try:
                for kern in ("dot", "mfma"):
                    os.environ["GQ8_W8A8_KERNEL"] = kern
                    rec[f"{kern}_us"] = round(timed(lambda i: (lambda s, w=wps[i % n]: gq8.gq8_w8a8_gemm(
                        xq, xs, w, wsc, out, M, N, K, wsp, nb, s)), n), 3)
            finally:
                if prev is None:
                    os.environ.pop("GQ8_W8A8_KERNEL", None)
                else:
                    os.environ["GQ8_W8A8_KERNEL"] = prev
            emit(rec)
            del wps


def bench_moe(torch, gq8, synth, dev, timed, emit):
    from gemm_q8_amd.device import to_dev
    # routed MoE: 512 experts, T=4, top-8, D=2048, F=512
    m = setup_moe(torch, gq8, synth, dev)
    T, E, topk, D, F = m["T"], m["E"], m["topk"], m["D"], m["F"]
    gu_b, dn_b, n, agus, adns = m["gu_b"], m["dn_b"], m["n"], m["agus"], m["adns"]
    inp, ids, wts, xq, xd, nb, wsp, out = (m["inp"], m["ids"], m["wts"], m["xq"], m["xd"], m["nb"],
                                           m["ws"], m["out"])
    U = len(m["routed"])
    us = timed(lambda i: (lambda s, a=agus[i % n], b=adns[i % n]: gq8.gq8_moe_q8_0_routed(
        xq, xd, ids, wts, a, b, out, T, topk, E, D, F, wsp, nb, s)), n, reps=50)
    emit({"workload": "routed MoE T=4 E=512 top-8 D=2048 F=512", "unique_experts": U,
          "us_per_call": round(us, 3), "weight_GBps": round(U * (gu_b + dn_b) / us / 1e3, 1)})
    # the same on the bf16 input: q8_1 quantization fused into the gate/up kernel, against the
    # quantize call followed by the routed call
    xb = to_dev(inp["x"])
    us = timed(lambda i: (lambda s, a=agus[i % n], b=adns[i % n]: gq8.gq8_moe_q8_0_routed_bf16(
        xb, ids, wts, a, b, out, T, topk, E, D, F, wsp, nb, s)), n, reps=50)
    emit({"workload": "routed MoE on the bf16 input (q8_1 fused) T=4 E=512 top-8 D=2048 F=512",
          "unique_experts": U, "us_per_call": round(us, 3), "weight_GBps": round(U * (gu_b + dn_b) / us / 1e3, 1)})

    for flags, name in ((gq8.MOE_H_Q8_1, "routed MoE, down read on q8_1(h)"),
                        (gq8.MOE_X_BF16 | gq8.MOE_H_Q8_1, "routed MoE on the bf16 input, down read on q8_1(h)")):
        xx, xs = (xb, None) if flags & gq8.MOE_X_BF16 else (xq, xd)
        us = timed(lambda i: (lambda s, a=agus[i % n], b=adns[i % n]: gq8.gq8_moe_q8_0_routed_flags(
            xx, xs, ids, wts, a, b, out, T, topk, E, D, F, flags, wsp, nb, s)), n, reps=50)
        emit({"workload": name + " T=4 E=512 top-8 D=2048 F=512", "unique_experts": U,
              "us_per_call": round(us, 3), "weight_GBps": round(U * (gu_b + dn_b) / us / 1e3, 1)})

    # the down weights in the tiled layout (bitwise the same outputs)
    adns_t = tiled_down_arenas(torch, gq8, m)
    for flags, name in ((gq8.MOE_DOWN_TILED, "routed MoE, down weights tiled"),
                        (gq8.MOE_X_BF16 | gq8.MOE_DOWN_TILED, "routed MoE on the bf16 input, down weights tiled"),
                        (gq8.MOE_H_Q8_1 | gq8.MOE_DOWN_TILED, "routed MoE, down read on q8_1(h), down weights tiled")):
        xx, xs = (xb, None) if flags & gq8.MOE_X_BF16 else (xq, xd)
        us = timed(lambda i: (lambda s, a=agus[i % n], b=adns_t[i % n]: gq8.gq8_moe_q8_0_routed_flags(
            xx, xs, ids, wts, a, b, out, T, topk, E, D, F, flags, wsp, nb, s)), n, reps=50)
        emit({"workload": name + " T=4 E=512 top-8 D=2048 F=512", "unique_experts": U,
              "us_per_call": round(us, 3), "weight_GBps": round(U * (gu_b + dn_b) / us / 1e3, 1)})
    del adns_t

    def two_calls(s, a, b):
        gq8.gq8_q8_1_quantize(xb, T, D, xq, xd, None, s)
        gq8.gq8_moe_q8_0_routed(xq, xd, ids, wts, a, b, out, T, topk, E, D, F, wsp, nb, s)
    us = timed(lambda i: (lambda s, a=agus[i % n], b=adns[i % n]: two_calls(s, a, b)), n, reps=50)
    emit({"workload": "q8_1 quantize + routed MoE T=4 E=512 top-8 D=2048 F=512",
          "unique_experts": U, "us_per_call": round(us, 3), "weight_GBps": round(U * (gu_b + dn_b) / us / 1e3, 1)})


def probe_sweep(torch, gq8, dev, stream, report, sizes=(4_456_448, 5_570_560, 6_291_456, 8_388_608,
                                                        10_485_760, 33_554_432)):
    """The read probe over launch shapes at the byte counts of the reads: loads per lane 1/2/4/8,
    256/512/1024 threads, one work-group per chunk or a fixed grid of 1, 2, 4 or 8 work-groups per
    CU striding over the chunks, non-temporal or plain loads; graphs of back-to-back launches over
    rotated buffers (>= 640 MiB). One JSON line per (size, shape); the fastest shape per size is
    logged."""
    cus = gq8.gq8_device_cus()
    lines = []
    for nbytes in sizes:
        n = n_sets_for(nbytes)
        bufs = [torch.ones(nbytes, dtype=torch.uint8, device=dev) for _ in range(n)]
        sink = torch.empty(gq8.gq8_read_probe_sink_floats(nbytes), dtype=torch.float32, device=dev)
        best = None
        for lpt in (1, 2, 4, 8):
            for threads in (256, 512, 1024):
                for wg in (0, cus, 2 * cus, 4 * cus, 8 * cus):
                    for nt in (1, 0):
                        d = timed_dist(torch, stream, lambda i, lpt=lpt, threads=threads, wg=wg, nt=nt: (
                            lambda s, b=bufs[i % n]: gq8.gq8_read_probe_ex(b, nbytes, sink, lpt, threads, wg, nt, s)),
                            n, reps=5, min_calls=200)
                        r = {"workload": "read probe sweep", "bytes": nbytes, "loads_per_lane": lpt,
                             "threads": threads, "work_groups": wg or "one per chunk", "nontemporal": nt,
                             "us_median": round(d["median"], 3), "GBps": round(nbytes / d["median"] / 1e3, 1)}
                        lines.append(r)
                        if best is None or r["us_median"] < best["us_median"]:
                            best = r
        log("[probe sweep] best " + json.dumps(best))
        del bufs
    if report:
        with open(report, "w") as f:
            for r in lines:
                f.write(json.dumps(r) + "\n")
    return lines


def to_host_ids(ids):
    return ids.cpu().numpy().ravel().tolist()


# ------------------------------------------------------------------------------------ the five workloads

class ProbeCache:
    """Same-byte read-probe times: one call = gq8_read_probe launches of the given sizes in
    sequence (a read of two launches is compared with two probe launches), over rotated buffers
    (>= 640 MiB), timed like the reads. Median us per call, cached by the launch sizes."""

    def __init__(self, torch, gq8, dev, stream, reps):
        self.torch, self.gq8, self.dev, self.stream, self.reps = torch, gq8, dev, stream, reps
        self.cache = {}

    def us(self, sizes):
        key = tuple(int(b) for b in sizes)
        if key not in self.cache:
            torch, gq8 = self.torch, self.gq8
            n = n_sets_for(sum(key))
            bufs = [[torch.ones(b, dtype=torch.uint8, device=self.dev) for b in key] for _ in range(n)]
            sink = torch.empty(max(gq8.gq8_read_probe_sink_floats(b) for b in key),
                               dtype=torch.float32, device=self.dev)

            def fn(i):
                bs = bufs[i % n]

                def f(s):
                    for b, nb in zip(bs, key):
                        gq8.gq8_read_probe(b, nb, sink, s)
                return f
            self.cache[key] = timed_dist(torch, self.stream, fn, n, reps=self.reps)["median"]
            del bufs
        return self.cache[key]


def oracle_times(fn):
    """The C++ oracle (test infrastructure) timed on the host: fn(threads) runs the whole call,
    on one thread and on every host core, after a warm-up call; a call under 20 ms is taken three
    times and the fastest kept (thread start-up noise). Returns (us at 1 thread, us at all
    cores, cores)."""
    from oracle import c_oracle as C
    fn(0)                                                  # first-touch / allocation warm-up

    def best(th):
        ts = []
        while len(ts) < 3 and (not ts or min(ts) < 0.02):
            t0 = time.perf_counter()
            fn(th)
            ts.append(time.perf_counter() - t0)
        return min(ts)
    return best(1) * 1e6, best(0) * 1e6, C.threads_available()


def config_record(cfg, workload, shape, d, wbytes, probe_us, orc, orc_sample):
    gbs = wbytes / d["median"] / 1e3
    r = {"config": cfg, "workload": workload, **shape,
         "us_median": round(d["median"], 3), "us_p90": round(d["p90"], 3), "us_mean": round(d["mean"], 3),
         "weight_bytes": int(wbytes), "weight_GBps": round(gbs, 1),
         "frac_of_8TBps": round(gbs / HBM_PEAK_GBS, 4),
         "probe_us": round(probe_us, 3), "frac_of_probe": round(probe_us / d["median"], 4)}
    if orc is not None:
        r["oracle_us_1thread"] = round(orc[0], 1)
        r["oracle_us_all_threads"] = round(orc[1], 1)
        r["oracle_threads"] = orc[2]
        r["oracle_sample"] = orc_sample
    return r


def setup_moe(torch, gq8, synth, dev, T=4, E=512, topk=8, D=2048, F=512, n_copies=8):
    """The routed-expert workload: routing from N(0,1) logits on the device, arenas of E experts
    (gate/up Q8_0 [2F, D] and down Q8_0 [D, F] each), n_copies copies rotated. Only the routed
    experts' bytes are ever read, so only they are drawn and quantized (the others are zero);
    every arena has the full E-expert size and layout."""
    from gemm_q8_amd.device import to_dev
    gu_b, dn_b = gq8.gq8_q8_0_bytes(2 * F, D), gq8.gq8_q8_0_bytes(D, F)
    inp = synth.moe_inputs(T=T, E=E, D=D)
    ids = torch.empty((T, topk), dtype=torch.int32, device=dev)
    wts = torch.empty((T, topk), dtype=torch.float32, device=dev)
    gq8.gq8_moe_route(to_dev(inp["logits"]), T, E, topk, ids, wts)
    routed = sorted(set(to_host_ids(ids)))
    agu = torch.zeros(E * gu_b, dtype=torch.uint8, device=dev)
    adn = torch.zeros(E * dn_b, dtype=torch.uint8, device=dev)
    for e in routed:
        w = synth.moe_expert_weights(e, D=D, F=F)
        gq8.gq8_q8_0_quantize(to_dev(w["gate_up"]), 2 * F, D, agu[e * gu_b:(e + 1) * gu_b])
        gq8.gq8_q8_0_quantize(to_dev(w["down"]), D, F, adn[e * dn_b:(e + 1) * dn_b])
    xq = torch.empty((T, D), dtype=torch.int8, device=dev)
    xd = torch.empty((T, D // 32), dtype=torch.int16, device=dev)
    gq8.gq8_q8_1_quantize(to_dev(inp["x"]), T, D, xq, xd, None)
    nb = gq8.gq8_moe_workspace_bytes(T, topk, D, F)
    return dict(T=T, E=E, topk=topk, D=D, F=F, gu_b=gu_b, dn_b=dn_b, inp=inp, ids=ids, wts=wts,
                routed=routed, agus=[agu] + [agu.clone() for _ in range(n_copies - 1)],
                adns=[adn] + [adn.clone() for _ in range(n_copies - 1)], n=n_copies, xq=xq, xd=xd,
                nb=nb, ws=torch.empty(nb, dtype=torch.uint8, device=dev),
                out=torch.empty((T, D), dtype=torch.int16, device=dev))


def tiled_down_arenas(torch, gq8, m):
    """The down arenas of setup_moe in the tiled layout (gq8_q8_0_tile16: same size and expert
    stride, quants in 1 KiB operand-order tiles), one per rotated copy."""
    out = []
    for a in m["adns"]:
        t = torch.empty_like(a)
        gq8.gq8_q8_0_tile16(a, m["D"], m["F"], m["E"], t)
        out.append(t)
    return out


def bench_configs(torch, gq8, synth, dev, stream, hc_dist, reps, hc_dist_tiled=None, with_oracle=True,
                  gemv_ts=(1, 2, 4, 8, 16)):
    """One record per workload shape of the five configurations: median / p90 / mean us per call
    (graphs of back-to-back calls over rotated weight copies, inputs in HBM), weight GB/s, the
    fraction of 8 TB/s and of the same-byte read probe, and the oracle's time on the host."""
    from gemm_q8_amd.device import q8_0_from_f32, to_dev, workspace
    from oracle import c_oracle as C
    from oracle.q8 import quantize_q8_0, quantize_q8_1_bf16
    probe = ProbeCache(torch, gq8, dev, stream, reps)
    recs = []

    def emit(r):
        recs.append(r)
        log("[config] " + json.dumps(r))

    # 1: Q8_0 GEMV N = 1024, K = 4096 (T = 1 is the configuration; the metric spans T = 1..16)
    d = synth.q8_0_gemv_inputs(T=16)
    w0 = q8_0_from_f32(to_dev(d["w"]))
    n = n_sets_for(w0.numel())
    wset = [w0] + [w0.clone() for _ in range(n - 1)]
    b = quantize_q8_0(d["w"]) if with_oracle else None
    for T in gemv_ts:
        x = to_dev(np.ascontiguousarray(d["x"][:T]))
        y = torch.empty((T, 1024), dtype=torch.float32, device=dev)
        nb = gq8.gq8_workspace_bytes(gq8.OP_Q8_0_GEMV, T, 1024, 4096)
        wsp = workspace(nb)
        dist = timed_dist(torch, stream, lambda i, T=T, x=x, y=y, nb=nb, wsp=wsp: (
            lambda s, w=wset[i % n]: gq8.gq8_q8_0_gemv(w, x, y, T, 1024, 4096, wsp, nb, s)), n, reps)
        xs = d["x"][:T]
        orc = oracle_times(lambda th: C.q8_0_gemv(b, xs, threads=th)) if with_oracle else None
        emit(config_record(1, "Q8_0 GEMV N=1024 K=4096", {"T": T}, dist, w0.numel(),
                           probe.us([w0.numel()]), orc, "the whole call (C++ oracle, float64)"))
    del wset

    # 2: the HC pair (timed with the step's own graphs)
    pair_w = 2 * (K_HC * N_LR + K_HC * N_LR // 32 * 2)
    if with_oracle:
        base = synth.hc_inputs(6)
        bd, bu = quantize_q8_0(base["w_down"]), quantize_q8_0(base["w_up"])
    for T in TS:
        if with_oracle:
            ins = synth.hc_inputs(T)

            def pair_oracle(th, ins=ins):
                lo, _, _ = C.hc_down(ins["R"], ins["w_norm"], bd, threads=th)
                C.hc_up(C.bf16_bits(lo.astype(np.float32)), bu, threads=th)
            orc = oracle_times(pair_oracle)
        else:
            orc = None
        emit(config_record(2, "HC pair: RMSNorm + Q8_0 down [320 x 16384], Q8_0 up [16384 x 320]",
                           {"T": T}, hc_dist[T], pair_w, probe.us([pair_w // 2, pair_w // 2]), orc,
                           "the whole call: down then up read (C++ oracle, float64)"))
    for T in sorted(hc_dist_tiled or {}):
        emit(config_record(2, "HC pair, up weights tiled (gq8_hc_q8_pair_tiled): RMSNorm + Q8_0 down "
                              "[320 x 16384], Q8_0 up [16384 x 320]",
                           {"T": T}, hc_dist_tiled[T], pair_w, probe.us([pair_w // 2, pair_w // 2]), None,
                           ""))

    # 3 and 4: W8A8
    for cfg, (M, N, K) in [(3, (16, 1536, 4096))] + [(4, (m, 2560, 4096)) for m in (1, 4, 8, 16, 32)] + \
                          [(4, (m, 4096, 2048)) for m in (1, 4, 8, 16, 32)]:
        dd = synth.w8a8_inputs(M, N, K)
        wp0 = torch.empty(gq8.gq8_w8a8_packed_bytes(K, N), dtype=torch.int8, device=dev)
        gq8.gq8_w8a8_pack(to_dev(dd["W"]), K, N, wp0)
        n = n_sets_for(wp0.numel())
        wps = [wp0] + [wp0.clone() for _ in range(n - 1)]
        xq, xs, wsc = to_dev(dd["xq"]), to_dev(dd["x_scale"]), to_dev(dd["w_scale"])
        out = torch.empty((M, N), dtype=torch.int16, device=dev)
        dist = timed_dist(torch, stream, lambda i: (lambda s, w=wps[i % n]: gq8.gq8_w8a8_gemm(
            xq, xs, w, wsc, out, M, N, K, None, 0, s)), n, reps)
        orc = (oracle_times(lambda th: C.w8a8_gemm(dd["xq"], dd["x_scale"], dd["W"], dd["w_scale"],
                                                   threads=th)) if with_oracle else None)
        emit(config_record(cfg, "W8A8 int8 x int8 -> int32 -> bf16", {"M": M, "N": N, "K": K}, dist,
                           N * K, probe.us([wp0.numel()]), orc, "the whole call (C++ oracle, int64)"))
        del wps

    # 5: routed MoE
    m = setup_moe(torch, gq8, synth, dev)
    T, E, topk, D, F = m["T"], m["E"], m["topk"], m["D"], m["F"]
    U = len(m["routed"])
    dist = timed_dist(torch, stream, lambda i: (lambda s, a=m["agus"][i % m["n"]], b=m["adns"][i % m["n"]]:
                                                 gq8.gq8_moe_q8_0_routed(m["xq"], m["xd"], m["ids"], m["wts"], a, b,
                                                                         m["out"], T, topk, E, D, F, m["ws"], m["nb"], s)),
                      m["n"], reps)
    orc = None
    if with_oracle:
        ids_h = m["ids"].cpu().numpy().astype(np.int64)
        p_h = m["wts"].cpu().numpy().astype(np.float64)
        cache = {e: (quantize_q8_0(synth.moe_expert_weights(e, D=D, F=F)["gate_up"]),
                     quantize_q8_0(synth.moe_expert_weights(e, D=D, F=F)["down"])) for e in m["routed"]}
        x81 = quantize_q8_1_bf16(m["inp"]["x"])
        prep = C.moe_prepare(x81, ids_h, p_h, lambda e: cache[e])
        orc = oracle_times(lambda th: C.moe_run(prep, threads=th))
    emit(config_record(5, "routed MoE: T=4, 512 experts, top-8, gate/up [1024 x 2048], down [2048 x 512]",
                       {"T": T, "E": E, "topk": topk, "unique_experts": U}, dist,
                       U * (m["gu_b"] + m["dn_b"]), probe.us([U * m["gu_b"], U * m["dn_b"]]), orc,
                       "the whole call (C++ oracle, float64; weights already quantized)"))
    # the same call on the down weights in the tiled layout (bitwise the same output)
    adns_t = tiled_down_arenas(torch, gq8, m)
    dist = timed_dist(torch, stream, lambda i: (lambda s, a=m["agus"][i % m["n"]], b=adns_t[i % m["n"]]:
                                                 gq8.gq8_moe_q8_0_routed_flags(m["xq"], m["xd"], m["ids"], m["wts"], a, b,
                                                                               m["out"], T, topk, E, D, F, gq8.MOE_DOWN_TILED,
                                                                               m["ws"], m["nb"], s)),
                      m["n"], reps)
    emit(config_record(5, "routed MoE, down weights tiled (gq8_q8_0_tile16): T=4, 512 experts, top-8, "
                          "gate/up [1024 x 2048], down [2048 x 512]",
                       {"T": T, "E": E, "topk": topk, "unique_experts": U}, dist,
                       U * (m["gu_b"] + m["dn_b"]), probe.us([U * m["gu_b"], U * m["dn_b"]]), orc,
                       "the whole call (C++ oracle, float64; weights already quantized)"))
    del m, adns_t
    return recs


# ------------------------------------------------------------------------------------ main

def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=42)
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="oracle time budget for cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--all-configs", action="store_true",
                    help="also the comparison reads and variants (BF16 pair, W8A8 on a bf16 x, MoE "
                         "options, the probe curve) on stderr and in --report")
    ap.add_argument("--probe-sweep", default="",
                    help="sweep the read probe's launch shapes and write the lines to this file, "
                         "then exit")
    ap.add_argument("--no-configs", action="store_true",
                    help="leave out the per-configuration records (the five workloads)")
    ap.add_argument("--only", default="probe,combine,hcbf16,gemv,w8a8,w8a8kern,moe",
                    help="with --all-configs: comma-separated subset of probe,combine,hcbf16,gemv,w8a8,w8a8kern,moe")
    ap.add_argument("--w8a8-ms", default="1,4,8,16,32", help="with --all-configs: W8A8 M values")
    ap.add_argument("--sweep-samples", type=int, default=0,
                    help="with --all-configs: samples of >= 400 calls per sweep line (0: the default, 6 for most; 1 keeps "
                         "profiler runs short)")
    ap.add_argument("--gemv-ts", default="1,2,4,8,16", help="token rows of the GEMV sweep")
    ap.add_argument("--report", default="bench_all.jsonl",
                    help="file for the --all-configs lines (JSON, one per line)")
    ap.add_argument("--reps", type=int, default=20,
                    help="replays of each per-call timing graph (per-T pair, down, up)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="also launch one device copy of this many MiB (for scaling PMC byte counters)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py: one GPU only (asked for --gpus {args.gpus}); "
              "the multi-GPU sharding is described, not run", file=sys.stderr)
        sys.exit(2)

    import torch
    from gemm_q8_amd import gq8, synth

    dev = "cuda:0"
    torch.cuda.set_device(0)
    stream = torch.cuda.Stream()
    log(f"[bench] device {torch.cuda.get_device_name(0)}, {gq8.gq8_device_cus()} CUs; lib {gq8.LIB_PATH}")
    if args.probe_sweep:
        probe_sweep(torch, gq8, dev, stream, args.probe_sweep)
        return

    h = setup_hc(torch, gq8, synth, dev)
    steps_per_graph = h["n_sets"] // len(TS)
    log(f"[bench] HC workload: {h['n_sets']} weight sets x {h['pair_bytes']} B, {steps_per_graph} steps per graph")
    gs = GraphSteps(torch, stream, hc_step_fns(gq8, h), steps_per_graph)
    gs.prepare(args.warmup).prepare(args.steps)

    # warmup, then exactly K timed steps bracketed by synchronizations
    gs.run(args.warmup)
    torch.cuda.synchronize()
    t = time_region(torch, stream, lambda: gs.run(args.steps))
    torch.cuda.synchronize()
    step_bytes = len(TS) * h["pair_bytes"]
    value = step_bytes * args.steps / t / 1e9
    ms_per_step = t / args.steps * 1e3
    log(f"[bench] {args.steps} steps in {t * 1e3:.3f} ms: {ms_per_step * 1e3:.2f} us/step, {value:.1f} GB/s")

    # per-T pair time (the step's own calls) and the separate down / up calls, each in graphs of
    # back-to-back calls over the rotated weight sets
    n = h["n_sets"]
    per_call = {}
    calls = {}
    kern = {}
    reps = max(1, args.reps)
    dist = {}
    hot = {}
    hc_dist = {}
    for T in TS:
        for kind, mk in (("pair", hc_pair_fn), ("down", hc_down_fn), ("up", hc_up_fn)):
            g = GraphSteps(torch, stream, lambda i, T=T, mk=mk: [mk(gq8, h, T, i)], n)
            g.run(n)
            # reps samples of one rotation each (n calls): the mean over all, and the median and
            # p90 of the per-sample per-call times
            ts = [time_region(torch, stream, lambda: g.run(n)) for _ in range(reps)]
            tk = sum(ts)
            k = kern.setdefault(kind, {"t": 0.0, "bytes": 0, "launches": 0})
            k["t"] += tk
            k["bytes"] += hc_kernel_bytes(kind, T) * n * reps
            k["launches"] += n * reps
            if kind == "pair":
                per_call[f"T{T}"] = round(tk / (n * reps) * 1e6, 3)
            else:
                calls[f"{kind}_T{T}"] = round(tk / (n * reps) * 1e6, 3)
        hc_dist[T] = timed_dist(torch, stream, lambda i, T=T: hc_pair_fn(gq8, h, T, i), n, reps)
        # hot cache: the same call on one weight set (5.6 MB per read stays in the 256 MB MALL)
        g = GraphSteps(torch, stream, lambda i, T=T: [hc_pair_fn(gq8, h, T, 0)], n)
        g.run(n)
        hot[f"T{T}"] = round(time_region(torch, stream, lambda: g.run(n * reps)) / (n * reps) * 1e6, 3)
    # the same pair with the up weights tiled (gq8_q8_0_tile16): a configuration record of its own
    hc_dist_tiled = {}
    if not args.no_configs:
        wus_t = []
        for w in h["wus"]:
            wt = torch.empty_like(w)
            gq8.gq8_q8_0_tile16(w, K_HC, N_LR, 1, wt)
            wus_t.append(wt)
        for T in TS:
            hc_dist_tiled[T] = timed_dist(torch, stream,
                                          lambda i, T=T: hc_pair_tiled_fn(gq8, h, wus_t, T, i), n, reps)
        del wus_t
    dom = "pair"
    # the roofline unit is the pair call, timed over the timed region itself: K steps of one
    # call per T, so the average call is t / (K * len(TS)) and its algorithmic bytes are the mean
    # of the T's
    n_calls = args.steps * len(TS)
    avg_us = t / n_calls * 1e6
    achieved = sum(hc_kernel_bytes("pair", T) for T in TS) * args.steps / t / 1e9
    dist = {f"T{T}": {"median": round(hc_dist[T]["median"], 3), "p90": round(hc_dist[T]["p90"], 3)}
            for T in TS}
    log(f"[bench] per-call pair us {per_call}; median/p90 {dist}; hot cache {hot}")
    log(f"[bench] per-call pair us {per_call}; calls: " + ", ".join(
        f"{k} {v['t'] / v['launches'] * 1e6:.3f} us" for k, v in kern.items()))

    if args.copy_probe_mib:
        nbytes = args.copy_probe_mib << 20
        a = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        with torch.cuda.stream(stream):
            b.copy_(a)
        torch.cuda.synchronize()
        log(f"[bench] copy probe: {nbytes} bytes read + {nbytes} written")

    page_pair = sum(PAGE_US[T] for T in TS)
    page_gbs = step_bytes / (page_pair * 1e-6) / 1e9
    result = {
        "metric": "achieved HBM GB/s (weight bytes/us) and us/call, Q8_0 & W8A8 decode, T=1..16",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": round(value / page_gbs, 3),
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": "fused RMSNorm + Q8_0 hyper-connection down read [320 x 16384] and Q8_0 up "
                        "read [16384 x 320], T in {1,4,6}",
            "T": list(TS),
            "weight_bytes_per_step": step_bytes,
            "weight_sets_rotated": h["n_sets"],
            "hipgraph": True,
            "us_per_pair": per_call,
            "us_per_pair_median_p90": dist,
            "us_per_pair_hot_cache": hot,
            "us_per_separate_call": calls,
            "hot_cache_note": "one weight set replayed: cache, not HBM (context only)",
            "lib_sha256": lib_sha256(gq8.LIB_PATH),
            "baseline_note": "vs_baseline divides by the HC-Q8 page's Arc Pro B70 Q8_0 read times "
                             "(24.7/29.3/34.4 us at T=1/4/6): another machine, context only",
        },
        "roofline": {
            "bound": "hbm",
            "kernel": "gq8_hc_q8_pair: hc_down_rows_kernel + hc_up_direct_kernel (T = 1); "
                      "hc_down_partial_kernel + hc_pair_up_kernel (T = 4); hc_down_partial_kernel "
                      "+ hc_down_combine_kernel + hc_up_direct_kernel (T = 6)",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": recorded_traffic(),
            "traffic_unit": "bytes per pair call (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-scaled)",
            "traffic_per_T": recorded_traffic(per_t=True),
            "traffic_note": "FETCH_SIZE counts every L2 fill from the memory side. At T = 1 the up "
                            "read's weights are filled twice: by the down launch's fetch-ahead "
                            "work-groups, then by the up read itself; the pair is faster for it, "
                            "which points to the second fill coming from the memory-side cache",
            "avg_call_us": round(avg_us, 3),
            "measured_over": f"the timed region: {args.steps} steps x {len(TS)} pair calls",
            # the same fraction per T (graphs of back-to-back calls of one T after the timed
            # region), and for the standalone down and up calls (their own kernels: partial sums +
            # combine kernel, and the up read alone), each over its own bytes
            "frac_per_T": {f"T{T}": round(hc_kernel_bytes("pair", T) / (per_call[f"T{T}"] * 1e3)
                                          / HBM_PEAK_GBS, 4) for T in TS},
            "separate_calls": {k: {"avg_us": round(v["t"] / v["launches"] * 1e6, 3),
                                   "achieved": round(v["bytes"] / v["t"] / 1e9, 2),
                                   "frac": round(v["bytes"] / v["t"] / 1e9 / HBM_PEAK_GBS, 4)}
                               for k, v in kern.items() if k != dom},
        },
    }
    if not args.no_configs:
        result["configs"] = bench_configs(torch, gq8, synth, dev, stream, hc_dist, reps, hc_dist_tiled,
                                          with_oracle=not args.no_cpu_baseline,
                                          gemv_ts=[int(t) for t in args.gemv_ts.split(",")])
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(synth, args.cpu_seconds)
    if args.all_configs:
        bench_other_configs(torch, gq8, synth, dev, stream, args.report, only=args.only.split(","),
                            w8a8_ms=[int(m) for m in args.w8a8_ms.split(",")],
                            gemv_ts=[int(t) for t in args.gemv_ts.split(",")],
                            samples=args.sweep_samples or None)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
