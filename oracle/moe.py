"""Routed-expert (MoE) decode with Q8_0 experts and a q8_1 input (oracle; test infrastructure).

EP page, "What changed": per layer, the routed expert ids and the q8_1 MoE
input go to the card that owns the experts; that card plans (groups the routed
entries by expert) and computes its entries, writing one output row per entry
into the owner's rows buffer (`parts_`); the owner then combines the rows. The
same page, "How it was checked", fixes what a plan must satisfy: every routed
entry appears exactly once. The defer page, "What it changes", combines expert
rows weighted by their routing weight.

The per-expert computation is the usual gated FFN: gate and up projections
(stored as one [2F, D] Q8_0 matrix, gate rows first), SiLU(gate) * up, then the
[D, F] Q8_0 down projection.

Readings taken where the pages are not explicit:
  * routing: softmax over all E logits, the top-k by probability in descending
    order (ties to the lower expert id), weights = those probabilities, not
    renormalised over the k;
  * plan order: experts ascending by id; within an expert, entries ascending by
    (token, slot);
  * gate/up blocks are integer dots of the Q8_0 weight quants with the q8_1
    input quants, scaled by both block scales; the down projection reads
    h = SiLU(g) * u unquantized (h is not re-quantized);
  * combine: y[t] = sum over slots j = 0..k-1 of p[t, j] * row[t, j], in slot order,
    stored as bf16.
  * the variant with h re-quantized (h_q8_1=True): h is rounded to fp32 (the precision the
    kernels keep it in), then quantized to q8_1 per 32-block with the input's rule (fp16
    amax / 127, fp32 quotient rounded half away from zero), and the down projection reads the
    dequantized d * q.
All real arithmetic is float64, integer dots int64.
"""
from __future__ import annotations

import numpy as np

from .numerics import fp16_to_f32
from .q8 import dequantize, quantize_q8_0


def route(logits, topk):
    """Returns (ids int64 [T, topk], p float64 [T, topk])."""
    l = np.asarray(logits, dtype=np.float64)
    z = np.exp(l - l.max(axis=1, keepdims=True))
    prob = z / z.sum(axis=1, keepdims=True)
    order = np.argsort(-prob, axis=1, kind="stable")[:, :topk]
    return order.astype(np.int64), np.take_along_axis(prob, order, axis=1)


def plan(ids):
    """Group routed entries by expert.

    Returns a list of (expert, [entry, ...]) with entry = t * topk + j, experts
    ascending and entries ascending within each expert.
    """
    ids = np.asarray(ids)
    T, topk = ids.shape
    groups = {}
    for t in range(T):
        for j in range(topk):
            groups.setdefault(int(ids[t, j]), []).append(t * topk + j)
    return [(e, groups[e]) for e in sorted(groups)]


def _gate_up(x81, t, gu):
    """Block-integer dots of expert rows with token t's q8_1 quants -> float64 [2F]."""
    qi = np.einsum("nbi,bi->nb", gu.q.astype(np.int64), x81.q[t].astype(np.int64))
    dw = fp16_to_f32(gu.d).astype(np.float64)
    dx = fp16_to_f32(x81.d[t]).astype(np.float64)
    return np.sum(dw * dx[None, :] * qi, axis=1)


def requantize_h(h):
    """h (float64 [F]) -> the real values d * q of its q8_1 form (float64 [F]), h first rounded to
    fp32."""
    return dequantize(quantize_q8_0(np.asarray(h, dtype=np.float32)[None, :]))[0]


def expert_rows(x81, t, gu, dn, h_q8_1=False):
    """One entry: returns (row float64 [D], S_row float64 [D]) where S_row = sum_k |d q h_k|
    (h_k the down read's input: h itself, or its q8_1 values for h_q8_1)."""
    F = gu.q.shape[0] // 2
    gu_v = _gate_up(x81, t, gu)
    g, u = gu_v[:F], gu_v[F:]
    h = g / (1.0 + np.exp(-g)) * u
    if h_q8_1:
        h = requantize_h(h)
    W = dequantize(dn)
    return W @ h, np.abs(W) @ np.abs(h)


def moe_forward(x81, ids, p, expert_blocks, h_q8_1=False):
    """y[t] = sum_j p[t, j] * expert_rows(ids[t, j]).

    x81: q8_1 blocks of the input [T, D]; expert_blocks(e) -> (gate_up Q8Blocks [2F, D],
    down Q8Blocks [D, F]).  Returns (y float64 [T, D], S float64 [T, D]).
    """
    ids = np.asarray(ids)
    T, topk = ids.shape
    D = x81.q.shape[1] * x81.q.shape[2]
    y = np.zeros((T, D))
    S = np.zeros((T, D))
    cache = {}
    for t in range(T):
        for j in range(topk):
            e = int(ids[t, j])
            if e not in cache:
                cache[e] = expert_blocks(e)
            r, s = expert_rows(x81, t, *cache[e], h_q8_1=h_q8_1)
            y[t] += p[t, j] * r
            S[t] += abs(p[t, j]) * s
    return y, S
