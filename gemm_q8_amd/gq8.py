"""Thin Python binding of libgq8.so (include/gq8.h), same names and argument order as the C ABI.

Argument marshalling only: device-pointer arguments accept a contiguous torch tensor on the GPU
(its data_ptr()), an int address, or None (NULL); the `_host` calls take C-contiguous numpy
arrays or contiguous CPU tensors instead (anything else raises ValueError before the call); `stream` defaults to torch's current stream on the current device.
A negative status raises GQ8Error. Every computation happens in the library's HIP kernels.

Importing this module loads libgq8.so and fails loudly if it has not been built
(python -m gemm_q8_amd.build) -- there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgq8.so")
if not os.path.exists(_LIB_PATH):
    raise ImportError(f"gemm_q8_amd: {_LIB_PATH} is missing; build it with `python -m gemm_q8_amd.build`")
_lib = ctypes.CDLL(_LIB_PATH)

LIB_PATH = _LIB_PATH

OK, EINVAL, ESHAPE, EALIGN, EWORKSPACE, ECAPTURE, EHIP, ENODEV = 0, -1, -2, -3, -4, -5, -6, -7
NOALLOC_SCRATCH_BYTES = 4 << 20
MOE_X_BF16, MOE_H_Q8_1, MOE_DOWN_TILED = 1, 2, 4
OP_Q8_0_GEMV, OP_HC_DOWN, OP_HC_UP, OP_W8A8, OP_HC_PAIR, OP_W8A8_BF16X = 1, 2, 3, 4, 5, 6

_P = ctypes.c_void_p
_I = ctypes.c_int
_I64 = ctypes.c_int64
_SZ = ctypes.c_size_t
_F = ctypes.c_float

# name -> (restype, argtypes), in include/gq8.h order
_SIGS = {
    "gq8_status_str": (ctypes.c_char_p, [_I]),
    "gq8_abi_version": (_I, []),
    "gq8_device_cus": (_I, [ctypes.POINTER(_I)]),
    "gq8_q8_0_bytes": (_SZ, [_I64, _I64]),
    "gq8_q8_0_quantize": (_I, [_P, _I, _I, _P, _P]),
    "gq8_q8_0_split_from_blocks": (_I, [_P, _I, _I, _P, _P]),
    "gq8_q8_0_tile16": (_I, [_P, _I, _I, _I, _P, _P]),
    "gq8_q8_1_quantize": (_I, [_P, _I, _I, _P, _P, _P, _P]),
    "gq8_workspace_bytes": (_SZ, [_I, _I, _I, _I]),
    "gq8_workspace_counter_bytes": (_SZ, [_I, _I, _I, _I]),
    "gq8_workspace_init": (_I, [_P, _SZ, _P]),
    "gq8_q8_0_gemv": (_I, [_P, _P, _P, _I, _I, _I, _P, _SZ, _P]),
    "gq8_hc_q8_down": (_I, [_P, _P, _P, _F, _P, _P, _I, _I, _I, _P, _SZ, _P]),
    "gq8_hc_q8_up": (_I, [_P, _P, _P, _I, _I, _I, _P, _SZ, _P]),
    "gq8_hc_q8_pair": (_I, [_P, _P, _P, _F, _P, _P, _P, _P, _I, _I, _I, _P, _SZ, _P]),
    "gq8_hc_q8_pair_tiled": (_I, [_P, _P, _P, _F, _P, _P, _P, _P, _I, _I, _I, _P, _SZ, _P]),
    "gq8_hc_q8_up_tiled": (_I, [_P, _P, _P, _I, _I, _I, _P, _SZ, _P]),
    "gq8_hc_q8_down_pending": (_I, [_P, _P, _P, _P, _F, _P, _P, _P, _I, _I, _I, _P, _SZ, _P]),
    "gq8_hc_q8_pair_pending": (_I, [_P, _P, _P, _P, _F, _P, _P, _P, _P, _P, _I, _I, _I, _P, _SZ, _P]),
    "gq8_hc_q8_pair_noalloc": (_I, [_P, _P, _P, _F, _P, _P, _P, _P, _I, _I, _I, _P]),
    "gq8_hc_bf16_pair": (_I, [_P, _P, _P, _F, _P, _P, _P, _P, _I, _I, _I, _P, _SZ, _P]),
    "gq8_w8a8_packed_bytes": (_SZ, [_I, _I]),
    "gq8_w8a8_pack": (_I, [_P, _I, _I, _P, _P]),
    "gq8_w8a8_gemm": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _P, _SZ, _P]),
    "gq8_w8a8_gemm_i32": (_I, [_P, _P, _P, _I, _I, _I, _P, _SZ, _P]),
    "gq8_quantize_per_token": (_I, [_P, _I, _I, _P, _P, _P]),
    "gq8_q8_0_quantize_host": (_I, [_P, _I, _I, _P]),
    "gq8_q8_0_split_from_blocks_host": (_I, [_P, _I, _I, _P]),
    "gq8_q8_1_quantize_host": (_I, [_P, _I, _I, _P, _P, _P]),
    "gq8_w8a8_pack_host": (_I, [_P, _I, _I, _P]),
    "gq8_workspace_check": (_I, [_I, _I, _I, _I, _P, _SZ, _P, _P]),
    "gq8_w8a8_gemm_bf16x": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _P, _SZ, _P]),
    "gq8_moe_route": (_I, [_P, _I, _I, _I, _P, _P, _P]),
    "gq8_moe_plan_words": (_SZ, [_I, _I]),
    "gq8_moe_plan": (_I, [_P, _I, _I, _I, _P, _P]),
    "gq8_moe_workspace_bytes": (_SZ, [_I, _I, _I, _I]),
    "gq8_moe_q8_0_routed": (_I, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _P, _SZ, _P]),
    "gq8_moe_q8_0_routed_bf16": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _P, _SZ, _P]),
    "gq8_moe_q8_0_routed_flags": (_I, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _P, _SZ, _P]),
    "gq8_read_probe_sink_floats": (_SZ, [_SZ]),
    "gq8_read_probe": (_I, [_P, _SZ, _P, _P]),
    "gq8_read_probe_ex": (_I, [_P, _SZ, _P, _I, _I, _I, _I, _P]),
}

for _name, (_res, _args) in _SIGS.items():
    _fn = getattr(_lib, _name)
    _fn.restype = _res
    _fn.argtypes = _args


class GQ8Error(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        super().__init__(f"{fn}: status {status} ({gq8_status_str(status)})")


def _dev(x):
    """Device address: a contiguous torch tensor on the GPU, an int address, or None."""
    if x is None or isinstance(x, int):
        return x
    if hasattr(x, "__array_interface__"):
        raise ValueError("a host (numpy) array was given where device memory is required")
    if not x.is_cuda:
        raise ValueError("a CPU tensor was given where device memory is required")
    if not x.is_contiguous():
        raise ValueError("device tensors must be contiguous")
    return x.data_ptr()


def _host(x):
    """Host address: a C-contiguous numpy array, a contiguous CPU torch tensor, an int, or None."""
    if x is None or isinstance(x, int):
        return x
    if hasattr(x, "__array_interface__"):
        if not x.flags["C_CONTIGUOUS"]:
            raise ValueError("host arrays must be C-contiguous")
        return x.__array_interface__["data"][0]
    if x.is_cuda:
        raise ValueError("a GPU tensor was given where host memory is required")
    if not x.is_contiguous():
        raise ValueError("host tensors must be contiguous")
    return x.data_ptr()


def _stream(s):
    if s is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(s, int):
        return s
    return s.cuda_stream


def _check(name, st):
    if st != OK:
        raise GQ8Error(name, st)
    return st


def gq8_status_str(status):
    return _lib.gq8_status_str(status).decode()


def gq8_abi_version():
    return _lib.gq8_abi_version()


def gq8_device_cus():
    c = _I(0)
    _check("gq8_device_cus", _lib.gq8_device_cus(ctypes.byref(c)))
    return c.value


def gq8_q8_0_bytes(rows, K):
    return _lib.gq8_q8_0_bytes(rows, K)


def gq8_q8_0_quantize(w, rows, K, w_split, stream=None):
    return _check("gq8_q8_0_quantize", _lib.gq8_q8_0_quantize(_dev(w), rows, K, _dev(w_split), _stream(stream)))


def gq8_q8_0_split_from_blocks(blocks34, rows, K, w_split, stream=None):
    return _check("gq8_q8_0_split_from_blocks",
                  _lib.gq8_q8_0_split_from_blocks(_dev(blocks34), rows, K, _dev(w_split), _stream(stream)))


def gq8_q8_0_tile16(w_split, rows, K, count, w_tiled, stream=None):
    return _check("gq8_q8_0_tile16",
                  _lib.gq8_q8_0_tile16(_dev(w_split), rows, K, count, _dev(w_tiled), _stream(stream)))


def gq8_q8_1_quantize(x_bf16, rows, K, q, d, s, stream=None):
    return _check("gq8_q8_1_quantize", _lib.gq8_q8_1_quantize(
        _dev(x_bf16), rows, K, _dev(q), _dev(d), _dev(s), _stream(stream)))


def gq8_workspace_bytes(op, rows, N, K):
    return _lib.gq8_workspace_bytes(op, rows, N, K)


def gq8_workspace_counter_bytes(op, rows, N, K):
    return _lib.gq8_workspace_counter_bytes(op, rows, N, K)


def gq8_workspace_init(ws, nbytes, stream=None):
    return _check("gq8_workspace_init", _lib.gq8_workspace_init(_dev(ws), nbytes, _stream(stream)))


def gq8_q8_0_gemv(w_split, x, y, T, N, K, ws, ws_bytes, stream=None):
    return _check("gq8_q8_0_gemv", _lib.gq8_q8_0_gemv(
        _dev(w_split), _dev(x), _dev(y), T, N, K, _dev(ws), ws_bytes, _stream(stream)))


def gq8_hc_q8_down(w_split, R, w_norm, eps, lo, rs_out, T, N, K, ws, ws_bytes, stream=None):
    return _check("gq8_hc_q8_down", _lib.gq8_hc_q8_down(
        _dev(w_split), _dev(R), _dev(w_norm), eps, _dev(lo), _dev(rs_out), T, N, K, _dev(ws), ws_bytes,
        _stream(stream)))


def gq8_hc_q8_up(w_split, lo, out, T, N, K, ws, ws_bytes, stream=None):
    return _check("gq8_hc_q8_up", _lib.gq8_hc_q8_up(
        _dev(w_split), _dev(lo), _dev(out), T, N, K, _dev(ws), ws_bytes, _stream(stream)))


def gq8_hc_q8_pair(w_down, R, w_norm, eps, w_up, lo, rs_out, out, T, Nlr, Khc, ws, ws_bytes,
                   stream=None):
    return _check("gq8_hc_q8_pair", _lib.gq8_hc_q8_pair(
        _dev(w_down), _dev(R), _dev(w_norm), eps, _dev(w_up), _dev(lo), _dev(rs_out), _dev(out),
        T, Nlr, Khc, _dev(ws), ws_bytes, _stream(stream)))


def gq8_hc_q8_up_tiled(w_tiled, lo, out, T, N, K, ws, ws_bytes, stream=None):
    return _check("gq8_hc_q8_up_tiled", _lib.gq8_hc_q8_up_tiled(
        _dev(w_tiled), _dev(lo), _dev(out), T, N, K, _dev(ws), ws_bytes, _stream(stream)))


def gq8_hc_q8_pair_tiled(w_down, R, w_norm, eps, w_up_tiled, lo, rs_out, out, T, Nlr, Khc, ws,
                         ws_bytes, stream=None):
    return _check("gq8_hc_q8_pair_tiled", _lib.gq8_hc_q8_pair_tiled(
        _dev(w_down), _dev(R), _dev(w_norm), eps, _dev(w_up_tiled), _dev(lo), _dev(rs_out),
        _dev(out), T, Nlr, Khc, _dev(ws), ws_bytes, _stream(stream)))


def gq8_hc_bf16_pair(w_down, R, w_norm, eps, w_up, lo, rs_out, out, T, Nlr, Khc, ws, ws_bytes,
                     stream=None):
    return _check("gq8_hc_bf16_pair", _lib.gq8_hc_bf16_pair(
        _dev(w_down), _dev(R), _dev(w_norm), eps, _dev(w_up), _dev(lo), _dev(rs_out), _dev(out),
        T, Nlr, Khc, _dev(ws), ws_bytes, _stream(stream)))


def gq8_w8a8_packed_bytes(K, N):
    return _lib.gq8_w8a8_packed_bytes(K, N)


def gq8_w8a8_pack(W, K, N, W_packed, stream=None):
    return _check("gq8_w8a8_pack", _lib.gq8_w8a8_pack(_dev(W), K, N, _dev(W_packed), _stream(stream)))


def gq8_w8a8_gemm(xq, x_scale, W_packed, w_scale, out, M, N, K, ws, ws_bytes, stream=None):
    return _check("gq8_w8a8_gemm", _lib.gq8_w8a8_gemm(
        _dev(xq), _dev(x_scale), _dev(W_packed), _dev(w_scale), _dev(out), M, N, K, _dev(ws), ws_bytes,
        _stream(stream)))


def gq8_w8a8_gemm_i32(xq, W_packed, acc, M, N, K, ws, ws_bytes, stream=None):
    return _check("gq8_w8a8_gemm_i32", _lib.gq8_w8a8_gemm_i32(
        _dev(xq), _dev(W_packed), _dev(acc), M, N, K, _dev(ws), ws_bytes, _stream(stream)))


def gq8_q8_0_quantize_host(w, rows, K, split_out):
    return _check("gq8_q8_0_quantize_host", _lib.gq8_q8_0_quantize_host(_host(w), rows, K, _host(split_out)))


def gq8_q8_0_split_from_blocks_host(blocks34, rows, K, split_out):
    return _check("gq8_q8_0_split_from_blocks_host",
                  _lib.gq8_q8_0_split_from_blocks_host(_host(blocks34), rows, K, _host(split_out)))


def gq8_q8_1_quantize_host(x_bf16, rows, K, q, d, s=None):
    return _check("gq8_q8_1_quantize_host",
                  _lib.gq8_q8_1_quantize_host(_host(x_bf16), rows, K, _host(q), _host(d), _host(s)))


def gq8_w8a8_pack_host(W, K, N, W_packed):
    return _check("gq8_w8a8_pack_host", _lib.gq8_w8a8_pack_host(_host(W), K, N, _host(W_packed)))


def gq8_workspace_check(op, rows, N, K, ws, nbytes, stream=None):
    """Number of non-zero words in a workspace's arrival-counter region (synchronizes the stream
    when the operation has counters)."""
    out = ctypes.c_int(-1)
    _check("gq8_workspace_check", _lib.gq8_workspace_check(
        op, rows, N, K, _dev(ws), nbytes, None if stream is None else _stream(stream),
        ctypes.addressof(out)))
    return out.value


def gq8_quantize_per_token(x, M, K, xq, xs, stream=None):
    return _check("gq8_quantize_per_token", _lib.gq8_quantize_per_token(
        _dev(x), M, K, _dev(xq), _dev(xs), _stream(stream)))


def gq8_w8a8_gemm_bf16x(x, W_packed, w_scale, out, xq_out, xs_out, M, N, K, ws, ws_bytes, stream=None):
    return _check("gq8_w8a8_gemm_bf16x", _lib.gq8_w8a8_gemm_bf16x(
        _dev(x), _dev(W_packed), _dev(w_scale), _dev(out), _dev(xq_out), _dev(xs_out), M, N, K,
        _dev(ws), ws_bytes, _stream(stream)))


def gq8_moe_route(logits, T, E, topk, ids, weights, stream=None):
    return _check("gq8_moe_route", _lib.gq8_moe_route(
        _dev(logits), T, E, topk, _dev(ids), _dev(weights), _stream(stream)))


def gq8_moe_plan_words(T, topk):
    return _lib.gq8_moe_plan_words(T, topk)


def gq8_moe_plan(ids, T, topk, E, plan, stream=None):
    return _check("gq8_moe_plan", _lib.gq8_moe_plan(_dev(ids), T, topk, E, _dev(plan), _stream(stream)))


def gq8_moe_workspace_bytes(T, topk, D, F):
    return _lib.gq8_moe_workspace_bytes(T, topk, D, F)


def gq8_moe_q8_0_routed(xq, xd, ids, weights, w_gate_up, w_down, out, T, topk, E, D, F, ws, ws_bytes,
                        stream=None):
    return _check("gq8_moe_q8_0_routed", _lib.gq8_moe_q8_0_routed(
        _dev(xq), _dev(xd), _dev(ids), _dev(weights), _dev(w_gate_up), _dev(w_down), _dev(out),
        T, topk, E, D, F, _dev(ws), ws_bytes, _stream(stream)))


def gq8_moe_q8_0_routed_bf16(x, ids, weights, w_gate_up, w_down, out, T, topk, E, D, F, ws, ws_bytes,
                             stream=None):
    return _check("gq8_moe_q8_0_routed_bf16", _lib.gq8_moe_q8_0_routed_bf16(
        _dev(x), _dev(ids), _dev(weights), _dev(w_gate_up), _dev(w_down), _dev(out),
        T, topk, E, D, F, _dev(ws), ws_bytes, _stream(stream)))


def gq8_moe_q8_0_routed_flags(x, xd, ids, weights, w_gate_up, w_down, out, T, topk, E, D, F, flags,
                              ws, ws_bytes, stream=None):
    return _check("gq8_moe_q8_0_routed_flags", _lib.gq8_moe_q8_0_routed_flags(
        _dev(x), _dev(xd), _dev(ids), _dev(weights), _dev(w_gate_up), _dev(w_down), _dev(out),
        T, topk, E, D, F, flags, _dev(ws), ws_bytes, _stream(stream)))


def gq8_read_probe_sink_floats(nbytes):
    return _lib.gq8_read_probe_sink_floats(nbytes)


def gq8_read_probe(src, nbytes, sink, stream=None):
    return _check("gq8_read_probe", _lib.gq8_read_probe(_dev(src), nbytes, _dev(sink), _stream(stream)))


def gq8_read_probe_ex(src, nbytes, sink, loads_per_lane, threads, work_groups, nontemporal,
                      stream=None):
    return _check("gq8_read_probe_ex", _lib.gq8_read_probe_ex(
        _dev(src), nbytes, _dev(sink), loads_per_lane, threads, work_groups, nontemporal,
        _stream(stream)))


def gq8_hc_q8_down_pending(w_split, R, P, w_norm, eps, R_out, lo, rs_out, T, N, K, ws, ws_bytes,
                           stream=None):
    return _check("gq8_hc_q8_down_pending", _lib.gq8_hc_q8_down_pending(
        _dev(w_split), _dev(R), _dev(P), _dev(w_norm), eps, _dev(R_out), _dev(lo), _dev(rs_out),
        T, N, K, _dev(ws), ws_bytes, _stream(stream)))


def gq8_hc_q8_pair_pending(w_down, R, P, w_norm, eps, w_up, R_out, lo, rs_out, out, T, Nlr, Khc, ws,
                           ws_bytes, stream=None):
    return _check("gq8_hc_q8_pair_pending", _lib.gq8_hc_q8_pair_pending(
        _dev(w_down), _dev(R), _dev(P), _dev(w_norm), eps, _dev(w_up), _dev(R_out), _dev(lo),
        _dev(rs_out), _dev(out), T, Nlr, Khc, _dev(ws), ws_bytes, _stream(stream)))


def gq8_hc_q8_pair_noalloc(w_down, R, w_norm, eps, w_up, lo, rs_out, out, T, Nlr, Khc, stream=None):
    return _check("gq8_hc_q8_pair_noalloc", _lib.gq8_hc_q8_pair_noalloc(
        _dev(w_down), _dev(R), _dev(w_norm), eps, _dev(w_up), _dev(lo), _dev(rs_out), _dev(out),
        T, Nlr, Khc, _stream(stream)))


def raw():
    """The ctypes library handle (for tests that check status codes without raising)."""
    return _lib
