"""The C++ oracle (oracle/c/gq8_oracle.cpp) through ctypes (test infrastructure).

The same definitions as the numpy oracle (q8, hc, w8a8, moe), written as plain loops in float64 /
int64 with a fixed k-ascending order per output and OpenMP over output rows, so one thread and all
host cores give bitwise the same result. It is used to time the oracle on the host (bench.py's
cpu_baseline) and is checked against the numpy oracle and its own pins (tests/test_oracle_c.py).
Each function takes the numpy oracle's block structures (Q8Blocks / Q81Blocks) and returns numpy
arrays; `threads` = 0 means all host cores.

The library is built by the repository's build step (python -m oracle.c.build); if it is
missing, importing this module builds it with the host compiler (a few seconds) and fails loudly
if that does not work.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from .q8 import Q8Blocks

_LIB = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c", "liboracle_c.so")
if not os.path.exists(_LIB):
    from .c.build import build as _build
    try:
        _build()
    except Exception as exc:  # noqa: BLE001
        raise ImportError(f"oracle: {_LIB} is missing and could not be built: {exc}") from exc
_lib = ctypes.CDLL(_LIB)

_P = ctypes.c_void_p
_I = ctypes.c_int
_L = ctypes.c_long
_D = ctypes.c_double
for _name, _args in {
    "orc_threads_available": [],
    "orc_f32_to_f16": [_P, _L, _P],
    "orc_f32_to_bf16": [_P, _L, _P],
    "orc_q8_0_quantize": [_P, _I, _I, _P, _P],
    "orc_q8_0_gemv": [_P, _P, _P, _I, _I, _I, _P, _P, _I],
    "orc_hc_up": [_P, _P, _P, _I, _I, _I, _P, _P, _I],
    "orc_hc_down": [_P, _P, _P, _P, _I, _I, _I, _D, _P, _P, _P, _I],
    "orc_w8a8": [_P, _P, _P, _P, _I, _I, _I, _P, _P, _I],
    "orc_moe_forward": [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _P, _P, _P, _I],
}.items():
    getattr(_lib, _name).argtypes = _args
    getattr(_lib, _name).restype = _I if _name == "orc_threads_available" else None


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _p(a):
    return a.ctypes.data_as(_P)


def threads_available():
    return int(_lib.orc_threads_available())


def f16_bits(x):
    x = _c(x, np.float32)
    out = np.empty(x.shape, np.uint16)
    _lib.orc_f32_to_f16(_p(x), x.size, _p(out))
    return out


def bf16_bits(x):
    x = _c(x, np.float32)
    out = np.empty(x.shape, np.uint16)
    _lib.orc_f32_to_bf16(_p(x), x.size, _p(out))
    return out


def quantize_q8_0(w):
    w = _c(w, np.float32)
    rows, K = w.shape
    d = np.empty((rows, K // 32), np.uint16)
    q = np.empty((rows, K // 32, 32), np.int8)
    _lib.orc_q8_0_quantize(_p(w), rows, K, _p(d), _p(q))
    return Q8Blocks(d=d, q=q)


def q8_0_gemv(blocks, x, threads=0):
    d, q = _c(blocks.d, np.uint16), _c(blocks.q, np.int8)
    x = _c(x, np.float32)
    T, K = x.shape
    N = d.shape[0]
    y, S = np.empty((T, N)), np.empty((T, N))
    _lib.orc_q8_0_gemv(_p(d), _p(q), _p(x), T, N, K, _p(y), _p(S), threads)
    return y, S


def hc_up(lo_bits, blocks, threads=0):
    d, q = _c(blocks.d, np.uint16), _c(blocks.q, np.int8)
    lo = _c(lo_bits, np.uint16)
    T, K = lo.shape
    N = d.shape[0]
    y, S = np.empty((T, N)), np.empty((T, N))
    _lib.orc_hc_up(_p(d), _p(q), _p(lo), T, N, K, _p(y), _p(S), threads)
    return y, S


def hc_down(R_bits, wnorm_bits, blocks, eps=1e-6, threads=0):
    d, q = _c(blocks.d, np.uint16), _c(blocks.q, np.int8)
    R, wn = _c(R_bits, np.uint16), _c(wnorm_bits, np.uint16)
    T, K = R.shape
    N = d.shape[0]
    lo, rs, S = np.empty((T, N)), np.empty(T), np.empty((T, N))
    _lib.orc_hc_down(_p(d), _p(q), _p(R), _p(wn), T, N, K, eps, _p(lo), _p(rs), _p(S), threads)
    return lo, rs, S


def w8a8_gemm(xq, x_scale, W, w_scale, threads=0):
    xq, W = _c(xq, np.int8), _c(W, np.int8)
    xs, ws = _c(x_scale, np.float32), _c(w_scale, np.float32)
    M, K = xq.shape
    N = W.shape[1]
    acc = np.empty((M, N), np.int64)
    out = np.empty((M, N), np.uint16)
    _lib.orc_w8a8(_p(xq), _p(xs), _p(W), _p(ws), M, N, K, _p(acc), _p(out), threads)
    return acc, out


def moe_prepare(x81, ids, p, expert_blocks):
    """The routed experts' blocks stacked for the C++ forward (marshalling, not the method)."""
    ids = _c(ids, np.int64)
    T, topk = ids.shape
    routed = sorted(set(ids.ravel().tolist()))
    slot = np.zeros(max(routed) + 1, np.int32)
    blocks = [expert_blocks(e) for e in routed]
    for u, e in enumerate(routed):
        slot[e] = u
    gu_d = _c(np.stack([b[0].d for b in blocks]), np.uint16)
    gu_q = _c(np.stack([b[0].q for b in blocks]), np.int8)
    dn_d = _c(np.stack([b[1].d for b in blocks]), np.uint16)
    dn_q = _c(np.stack([b[1].q for b in blocks]), np.int8)
    F = gu_d.shape[1] // 2
    D = dn_d.shape[1]
    return dict(T=T, topk=topk, D=D, F=F, ids=ids, slot=slot, gu_d=gu_d, gu_q=gu_q, dn_d=dn_d,
                dn_q=dn_q, xq=_c(x81.q.reshape(T, D), np.int8), xd=_c(x81.d, np.uint16),
                p=_c(p, np.float64))


def moe_run(prep, threads=0):
    T, topk, D, F = prep["T"], prep["topk"], prep["D"], prep["F"]
    y, S, h = np.empty((T, D)), np.empty((T, D)), np.empty((T * topk, F))
    _lib.orc_moe_forward(_p(prep["xq"]), _p(prep["xd"]), _p(prep["ids"]), _p(prep["p"]),
                         _p(prep["slot"]), _p(prep["gu_d"]), _p(prep["gu_q"]), _p(prep["dn_d"]),
                         _p(prep["dn_q"]), T, topk, D, F, _p(y), _p(S), _p(h), threads)
    return y, S


def moe_forward(x81, ids, p, expert_blocks, threads=0):
    """y[t] = sum_j p[t, j] * (down . SiLU(gate) * up)(expert ids[t, j]); expert_blocks(e) ->
    (gate_up Q8Blocks [2F, D], down Q8Blocks [D, F]). Returns (y, S) float64 [T, D]."""
    return moe_run(moe_prepare(x81, ids, p, expert_blocks), threads)
