"""Seeded synthetic inputs for the decode-time quantized matrix products.

This module only draws numbers: it holds none of the method's arithmetic (no
quantization, no products, no rounding of results). Both the product path's
callers (bench, tests) and the test oracle take their inputs from here, so the
two sides see the same values.

Every tensor comes from its own PCG64 stream, keyed by (seed, tensor name,
optional sub-index), so any one tensor can be regenerated alone: e.g. one
expert of a 512-expert arena without drawing the other 511.

Distributions follow the workloads the pages describe:
  * weights N(0, 0.02), activations N(0, 1) (fp32 or bf16)
  * RMSNorm weight N(1, 0.1) in bf16
  * int8 operands uniform on the integers -127..127, scales U(1e-3, 1e-2)
  * router logits N(0, 1)
bf16 values are made by dropping the low 16 bits of an fp32 draw (truncation):
a way of drawing bf16 numbers, not a rounding step of the method.
"""
from __future__ import annotations

import zlib

import numpy as np

__all__ = [
    "rng", "normal_f32", "uniform_f32", "int8_uniform", "bf16_normal",
    "bf16_bits_to_f32", "q8_0_gemv_inputs", "hc_inputs", "w8a8_inputs",
    "moe_inputs", "moe_expert_weights",
]


def _tag(name: str) -> int:
    return zlib.crc32(name.encode("utf-8")) & 0xFFFFFFFF


def rng(seed: int, name: str, *sub: int) -> np.random.Generator:
    """Independent generator for tensor `name` (and optional sub-indices)."""
    ss = np.random.SeedSequence([int(seed) & 0xFFFFFFFF, _tag(name), *[int(s) for s in sub]])
    return np.random.Generator(np.random.PCG64(ss))


def normal_f32(seed, name, shape, mean=0.0, std=1.0, *sub):
    g = rng(seed, name, *sub)
    x = g.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    if mean != 0.0:
        x += np.float32(mean)
    return x


def uniform_f32(seed, name, shape, lo, hi, *sub):
    g = rng(seed, name, *sub)
    return (np.float32(lo) + g.random(size=shape, dtype=np.float32) * np.float32(hi - lo)).astype(np.float32)


def int8_uniform(seed, name, shape, lo=-127, hi=127, *sub):
    g = rng(seed, name, *sub)
    return g.integers(lo, hi + 1, size=shape, dtype=np.int16).astype(np.int8)


def bf16_normal(seed, name, shape, mean=0.0, std=1.0, *sub):
    """bf16 bit patterns (uint16) of N(mean, std) draws, by truncation."""
    x = normal_f32(seed, name, shape, mean, std, *sub)
    return (x.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# --------------------------------------------------------------------------------------
# Workload recipes
# --------------------------------------------------------------------------------------

def q8_0_gemv_inputs(T=1, N=1024, K=4096, seed=0):
    """Q8_0 GEMV: fp32 weights W[N,K] ~ N(0,0.02) (quantized by the caller), x[T,K] ~ N(0,1)."""
    return {
        "w": normal_f32(seed, "gemv.w", (N, K), 0.0, 0.02),
        "x": normal_f32(seed, "gemv.x", (T, K), 0.0, 1.0),
    }


def hc_inputs(T, K=16384, N=320, seed=0):
    """Hyper-connection down/up read: R bf16 [T,K] ~ N(0,1), w_norm bf16 [K] ~ N(1,0.1),
    W_down fp32 [N,K] and W_up fp32 [K,N] ~ N(0,0.02) (quantized by the caller)."""
    return {
        "R": bf16_normal(seed, "hc.R", (T, K), 0.0, 1.0),
        "w_norm": bf16_normal(seed, "hc.w_norm", (K,), 1.0, 0.1),
        "w_down": normal_f32(seed, "hc.w_down", (N, K), 0.0, 0.02),
        "w_up": normal_f32(seed, "hc.w_up", (K, N), 0.0, 0.02),
    }


def hc_weights_bf16(K=16384, N=320, seed=0):
    """The hyper-connection weights of hc_inputs (same draws) as bf16 bit patterns, by
    truncation: W_down [N,K], W_up [K,N] (the BF16 comparison read)."""
    return {
        "w_down": bf16_normal(seed, "hc.w_down", (N, K), 0.0, 0.02),
        "w_up": bf16_normal(seed, "hc.w_up", (K, N), 0.0, 0.02),
    }


def w8a8_inputs(M, N, K, seed=0):
    """W8A8: x_q int8 [M,K], W int8 [K,N] (logical, k-major), scales U(1e-3,1e-2)."""
    return {
        "xq": int8_uniform(seed, "w8a8.xq", (M, K)),
        "x_scale": uniform_f32(seed, "w8a8.x_scale", (M,), 1e-3, 1e-2),
        "W": int8_uniform(seed, "w8a8.W", (K, N)),
        "w_scale": uniform_f32(seed, "w8a8.w_scale", (N,), 1e-3, 1e-2),
    }


def w8a8_bf16_inputs(M, N, K, seed=0):
    """W8A8 on a bf16 activation: x bf16 [M,K] ~ N(0,1) times a per-row factor U(0.05, 20) (rows
    of different magnitude), W int8 [K,N], w_scale U(1e-3,1e-2)."""
    rowf = uniform_f32(seed, "w8a8b.rowf", (M, 1), 0.05, 20.0)
    x = (normal_f32(seed, "w8a8b.x", (M, K)) * rowf).astype(np.float32)
    return {
        "x": (x.view(np.uint32) >> np.uint32(16)).astype(np.uint16),
        "W": int8_uniform(seed, "w8a8.W", (K, N)),
        "w_scale": uniform_f32(seed, "w8a8.w_scale", (N,), 1e-3, 1e-2),
    }


def moe_expert_weights(e, D=2048, F=512, seed=0):
    """Expert e's fp32 weights: gate/up [2F, D] (gate rows first) and down [D, F]."""
    return {
        "gate_up": normal_f32(seed, "moe.gate_up", (2 * F, D), 0.0, 0.02, e),
        "down": normal_f32(seed, "moe.down", (D, F), 0.0, 0.02, e),
    }


def moe_inputs(T=4, E=512, D=2048, seed=0):
    """Routed-expert inputs: router logits [T,E] ~ N(0,1), activations bf16 [T,D] ~ N(0,1)."""
    return {
        "logits": normal_f32(seed, "moe.logits", (T, E), 0.0, 1.0),
        "x": bf16_normal(seed, "moe.x", (T, D), 0.0, 1.0),
    }
