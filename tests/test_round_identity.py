"""Host check of the rounding shortcut the bf16-activation W8A8 kernels use: for fp32 y (the
rounded product x * inv), round half away from zero equals trunc(fl(y + copysign(0.5 - 2^-25, y))).
The per-token oracle applies the definition (trunc, then a step away from zero at a fractional
part >= 1/2); this compares the two on every fp32 in [0.25, 1), on the +-512-ulp neighbourhoods of
every integer and half-integer up to 128, and on their negatives. Below 0.25 both are 0."""
import numpy as np

C = np.float32(np.nextafter(np.float32(0.5), np.float32(0)))


def _shortcut(y):
    return np.trunc((y + np.copysign(C, y)).astype(np.float32))


def _definition(y):
    t = np.trunc(y)
    return np.where(np.abs(y - t) >= 0.5, t + np.sign(y), t)


def _check(u):
    y = u.astype(np.uint32).view(np.float32)
    for v in (y, -y):
        assert np.array_equal(_shortcut(v), _definition(v))


def test_bias_constant():
    assert C.view(np.uint32) == 0x3EFFFFFF and np.float64(C) == 0.5 - 2.0 ** -25


def test_every_float_in_quarter_to_one():
    lo, hi = np.float32(0.25).view(np.uint32), np.float32(1.0).view(np.uint32)
    for s in range(int(lo), int(hi), 1 << 22):
        _check(np.arange(s, min(s + (1 << 22), int(hi)), dtype=np.uint64))


def test_neighbourhoods_of_half_integers():
    centres = (np.arange(0, 257, dtype=np.float32) / np.float32(2))[1:]
    base = centres.view(np.uint32).astype(np.int64)
    u = (base[:, None] + np.arange(-512, 513)[None, :]).ravel()
    _check(u[u > 0])
