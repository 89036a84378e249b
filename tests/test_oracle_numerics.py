"""Pins for the oracle's number formats: known encodings, ties, and an independent library (torch)."""
import numpy as np
import pytest

from oracle.numerics import bf16_bits, bf16_to_f32, bf16_ulp, fp16_bits, fp16_to_f32, round_half_away


def test_fp16_known_encodings():
    vals = np.array([1.0, -2.0, 65504.0, 2.0 ** -24, 2.0 ** -14, 0.0, 0.5], dtype=np.float32)
    want = [0x3C00, 0xC000, 0x7BFF, 0x0001, 0x0400, 0x0000, 0x3800]
    assert fp16_bits(vals).tolist() == want
    # ties to even: 1 + 2^-11 is halfway between 1 and 1 + 2^-10
    assert fp16_bits(np.float32(1 + 2.0 ** -11)) == 0x3C00
    assert fp16_bits(np.float32(1 + 3 * 2.0 ** -11)) == 0x3C02
    assert fp16_to_f32(np.uint16(0x3555)) == np.float32(0.333251953125)


def test_bf16_known_encodings_and_ties():
    assert bf16_bits(np.float32(1.0)) == 0x3F80
    assert bf16_bits(np.float32(257.0)) == 0x4380   # tie between 256 and 258 -> even (256)
    assert bf16_bits(np.float32(259.0)) == 0x4382   # tie between 258 and 260 -> even (260)
    assert bf16_bits(np.float32(258.0)) == 0x4381
    assert bf16_to_f32(np.uint16(0x4382)) == np.float32(260.0)


def test_bf16_matches_torch_rounding():
    torch = pytest.importorskip("torch")
    g = np.random.default_rng(1)
    x = g.standard_normal(200000).astype(np.float32) * np.float32(37.0)
    # force exact ties on a slice: low 16 bits = 0x8000
    u = x.view(np.uint32).copy()
    u[:5000] = (u[:5000] & np.uint32(0xFFFF0000)) | np.uint32(0x8000)
    x = u.view(np.float32)
    ours = bf16_bits(x)
    theirs = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, theirs)


def test_round_half_away():
    v = np.array([0.5, -0.5, 1.5, 2.5, -2.5, 0.49999997, -0.49999997, 126.5, -127.49998, 8388607.5],
                 dtype=np.float32)
    assert round_half_away(v).tolist() == [1, -1, 2, 3, -3, 0, 0, 127, -127, 8388608]


def test_bf16_ulp_known_spacings():
    """bf16 keeps 8 significant bits: the spacing in [2^e, 2^(e+1)) is 2^(e-7); below the smallest
    normal the spacing of the smallest normal binade is used."""
    v = np.array([1.0, 1.99, 2.0, -3.0, 0.75, 2.0 ** -126, 0.0, 2.0 ** -130, 3.0e38], np.float64)
    want = [2.0 ** -7, 2.0 ** -7, 2.0 ** -6, 2.0 ** -6, 2.0 ** -8, 2.0 ** -133, 2.0 ** -133,
            2.0 ** -133, 2.0 ** 120]
    assert bf16_ulp(v).tolist() == want


def test_bf16_ulp_is_the_gap_to_the_next_bf16():
    """For every positive normal finite bf16 value b (all 32,512 bit patterns below the largest),
    bf16_ulp(b) equals the distance to the next bf16 up (bit pattern + 1): the spacing as the
    format itself defines it."""
    bits = np.arange(0x0080, 0x7F7F, dtype=np.uint32)
    b = bf16_to_f32(bits.astype(np.uint16)).astype(np.float64)
    nxt = bf16_to_f32((bits + 1).astype(np.uint16)).astype(np.float64)
    assert np.array_equal(bf16_ulp(b), nxt - b)
    assert np.array_equal(bf16_ulp(-b), nxt - b)
