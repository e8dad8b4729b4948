"""Pins of the oracle's MXFP4 decode.

The decode rule is the one on the vLLM page "flashinfer_moe_ep.py"
(_E2M1_LUT, _dequant_fp4_ue8m0_gran32): LUT value of the nibble (low nibble =
even element) times the float whose bit pattern is scale<<23.  The pins are
(a) the LUT as printed on that page (tests/golden/e2m1_lut.txt), (b) the e2m1
format definition written out independently (sign, 2-bit exponent with bias 1,
1-bit mantissa, subnormal at exponent 0), exhaustively over all 256 bytes, and
(c) the scale's bit-pattern reading done with numpy bit casts."""
import os

import numpy as np
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _lut():
    with open(os.path.join(GOLDEN, "e2m1_lut.txt")) as f:
        return [float(l) for l in f if l.strip() and not l.startswith("#")]


def _e2m1_from_format(code: int) -> float:
    sign = -1.0 if code & 8 else 1.0
    exp = (code >> 1) & 3
    man = code & 1
    if exp == 0:
        return sign * 0.5 * man
    return sign * 2.0 ** (exp - 1) * (1.0 + 0.5 * man)


def _scale_from_bits(s: int) -> float:
    return float(np.array([s << 23], dtype=np.uint32).view(np.float32)[0])


def test_page_lut_matches_format_definition():
    lut = _lut()
    assert len(lut) == 16
    for c in range(16):
        assert lut[c] == _e2m1_from_format(c)
        assert np.signbit(lut[c]) == bool(c & 8)


def test_scale_byte_rule():
    for s in range(256):
        got = oracle.e8m0_scale(s)
        want = _scale_from_bits(s)
        assert got == want, s
    assert oracle.e8m0_scale(0) == 0.0
    assert oracle.e8m0_scale(255) == float("inf")
    assert oracle.e8m0_scale(127) == 1.0


def test_exhaustive_byte_decode():
    lut = _lut()
    for s in (1, 60, 120, 125, 127, 130, 200, 254):
        packed = np.arange(256, dtype=np.uint8).reshape(1, 256)
        scales = np.full((1, 16), s, dtype=np.uint8)
        K = 512
        for b in range(256):
            lo = oracle.mxfp4_value(packed, scales, 0, K, 2 * b)
            hi = oracle.mxfp4_value(packed, scales, 0, K, 2 * b + 1)
            assert lo == lut[b & 15] * _scale_from_bits(s)
            assert hi == lut[b >> 4] * _scale_from_bits(s)


def test_scale_blocks_are_32_wide_along_k():
    packed = np.full((2, 32), 0x22, dtype=np.uint8)   # every element = code 2 = 1.0
    scales = np.array([[127, 128], [126, 130]], dtype=np.uint8)
    d = oracle.mxfp4_dequant(packed, scales)
    assert np.all(d[0, :32] == 1.0) and np.all(d[0, 32:] == 2.0)
    assert np.all(d[1, :32] == 0.5) and np.all(d[1, 32:] == 8.0)


def test_decoded_values_exact_in_bf16():
    # Every e2m1 value times 2^(s-127) is a bf16 number: the
    # decode can be fed to a bf16 path without rounding.
    # (s <= 252: at 253 and 254 the largest codes overflow a float's range.)
    for s in (1, 2, 100, 127, 200, 251, 252):
        vals = torch.tensor([_e2m1_from_format(c) * 2.0 ** (s - 127) for c in range(16)],
                            dtype=torch.float64)
        assert torch.equal(vals.to(torch.bfloat16).to(torch.float64), vals)
