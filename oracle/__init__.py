"""CPU oracle for the decode-time quantized matrix products (test infrastructure).

This package is TEST INFRASTRUCTURE. Only `tests/`, `__graft_entry__.smoke()` and
the `cpu_baseline` leg of `bench.py` may import it. The product path (the HIP
library under `gemm_q8_amd/` and its Python binding) never imports, links or
calls anything here, and nothing here imports the product path: the two share
no code. The only common module is `gemm_q8_amd.synth`, which draws the seeded
inputs and holds none of the method's arithmetic.

Everything is plain numpy: integer work in int64, real arithmetic in float64,
except where the method fixes a narrower precision for a decision (the
quantizers take their rounding decisions in fp32, as the kernels do; the W8A8
epilogue is specified in fp32). The oracle never reads the library's packed
weight layouts: it works on its own block structures, so a parity test also
covers the library's converters and packers.

Pages cited (by title and section):
  * "sycl: STRATA_HC_Q8=1 reads the Q8_0 hyper-connection projections" (PR #2810)
    -- the "HC-Q8 page".
  * "sycl: --expert-parallel-device N, two Arc cards compute each layer's
    experts together" (PR #1798) -- the "EP page".
  * "verify: STRATA_VERIFY_DEFER_CPU_BELOW=<w>" (PR #2690) -- the "defer page".
  * "INT8 W8A8 GEMM -- Decode (M <= 32) -- gfx928 / SGLang TP4" -- the
    "W8A8 page".

Modules:
  numerics  fp16 / bf16 conversions and round-half-away-from-zero
  q8        Q8_0 and q8_1 block quantizers, Q8_0 matrix-vector product
  hc        fused RMSNorm + Q8_0 down read and the Q8_0 up read
  w8a8      int8 x int8 -> int32 product with the fp32 scale epilogue
  moe       routing, the expert plan and the routed-expert Q8_0 forward
"""
from . import numerics, q8, hc, w8a8, moe  # noqa: F401
