"""Device-memory plumbing around the binding: numpy <-> torch device tensors, quantized weight
buffers and initialised workspaces. Memory only; every computation is a libgq8 call."""
from __future__ import annotations

import numpy as np
import torch

from . import gq8

_TORCH_OF = {
    np.dtype(np.float32): torch.float32,
    np.dtype(np.int8): torch.int8,
    np.dtype(np.int32): torch.int32,
    np.dtype(np.uint8): torch.uint8,
}


def to_dev(a: np.ndarray, device="cuda") -> torch.Tensor:
    """Upload a numpy array; uint16 arrays (bf16 / fp16 bit patterns) become int16 tensors."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        t = torch.from_numpy(a.view(np.int16))
    else:
        t = torch.from_numpy(a)
    return t.to(device)


def to_host(t: torch.Tensor, dtype=None) -> np.ndarray:
    a = t.detach().cpu().contiguous()
    if a.dtype in (torch.bfloat16, torch.float16):
        a = a.view(torch.int16)
    a = a.numpy()
    if dtype is not None:
        a = a.view(dtype)
    return a


def empty_bytes(nbytes: int, device="cuda") -> torch.Tensor:
    return torch.empty(max(int(nbytes), 16), dtype=torch.uint8, device=device)


def q8_0_from_f32(w: torch.Tensor, stream=None) -> torch.Tensor:
    """Quantize device fp32 rows [rows, K] into a new split-layout Q8_0 buffer (uint8)."""
    rows, K = w.shape
    out = empty_bytes(gq8.gq8_q8_0_bytes(rows, K), w.device)
    gq8.gq8_q8_0_quantize(w, rows, K, out, stream)
    return out


def q8_0_split_views(buf: torch.Tensor, rows: int, K: int):
    """(quants int8 [rows, K], scales fp16 bits int16 [rows, K/32]) views of a split buffer."""
    q = buf[: rows * K].view(torch.int8).view(rows, K)
    d = buf[rows * K: rows * K + rows * (K // 32) * 2].view(torch.int16).view(rows, K // 32)
    return q, d


def workspace(nbytes: int, device="cuda", stream=None):
    """An initialised workspace of `nbytes` (None when no workspace is needed)."""
    if nbytes == 0:
        return None
    ws = empty_bytes(nbytes, device)
    gq8.gq8_workspace_init(ws, nbytes, stream)
    return ws
