"""Pins for the oracle's number formats and exact dequantisation (CPU only)."""

import math

import numpy as np
import pytest
import torch

import oracle
from oracle import formats as F


# The 16 e2m1 values, code 0..15, as the OCP microscaling FP4 element is
# defined: sign, exponent bias 1, one mantissa bit, exponent 0 subnormal.
E2M1_TABLE = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0,
              -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0]


def test_e2m1_all_codes():
    got = oracle.e2m1_value(np.arange(16))
    assert got.tolist() == E2M1_TABLE
    assert math.copysign(1.0, got[8]) == -1.0          # code 8 is -0


def test_e4m3fn_all_codes_against_torch():
    codes = np.arange(256)
    got = oracle.e4m3fn_value(codes)
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.flatnonzero(nan).tolist() == [0x7F, 0xFF]
    assert np.array_equal(got[~nan], ref[~nan])
    assert got[0x38] == 1.0 and got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9
    assert got[0x30] == 0.5 and got[0x3F] == 1.875 and got[0x08] == 2.0 ** -6


def test_bf16_and_fp16_bits_against_torch():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    t = torch.from_numpy(bits.view(np.int16).copy())
    ref_bf = t.view(torch.bfloat16).to(torch.float64).numpy()
    ref_h = t.view(torch.float16).to(torch.float64).numpy()
    got_bf = oracle.bf16_bits_to_f64(bits)
    got_h = oracle.fp16_bits_to_f64(bits)
    for got, ref in ((got_bf, ref_bf), (got_h, ref_h)):
        nan = np.isnan(ref)
        assert np.array_equal(np.isnan(got), nan)
        assert np.array_equal(got[~nan], ref[~nan])


def test_rne_bf16_matches_torch_on_float32_inputs():
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 2 ** 32, size=200000, dtype=np.uint64).astype(np.uint32)
    # force many exact ties: low 16 bits = 0x8000
    bits[:20000] = (bits[:20000] & 0xFFFF0000) | 0x8000
    x = bits.view(np.float32)
    x = x[np.isfinite(x)]
    ref = torch.from_numpy(x.copy()).to(torch.bfloat16).to(torch.float64).numpy()
    got = oracle.rne_bf16(x.astype(np.float64))
    assert np.array_equal(got, ref)


def test_rne_bf16_rounds_once_from_float64():
    # 1 + 2**-8 + 2**-30 lies just above the midpoint of 1 and 1 + 2**-7:
    # one rounding gives 1 + 2**-7; rounding through float32 first loses the
    # 2**-30 and then ties to even at 1.0.
    assert oracle.rne_bf16(1.0 + 2 ** -8 + 2 ** -30) == 1.0 + 2 ** -7
    assert oracle.rne_bf16(1.0 + 2 ** -8) == 1.0                     # tie to even
    assert oracle.rne_bf16(1.0 + 3 * 2 ** -8) == 1.0 + 2 ** -6        # tie to even
    assert oracle.rne_bf16(-(1.0 + 2 ** -8 + 2 ** -30)) == -(1.0 + 2 ** -7)
    assert oracle.rne_bf16(2.0 ** -134) == 0.0                        # subnormal tie
    assert oracle.rne_bf16(3 * 2.0 ** -134) == 2.0 ** -132
    top = (2.0 - 2 ** -7) * 2.0 ** 127
    assert oracle.rne_bf16(top) == top
    assert oracle.rne_bf16(2.0 ** 128 - 2.0 ** 119) == math.inf       # midpoint -> even (overflow)
    assert oracle.rne_bf16(2.0 ** 128 - 2.0 ** 119 - 2.0 ** 90) == top
    assert math.copysign(1.0, oracle.rne_bf16(-0.0)) == -1.0


def test_unpack_nibbles_order():
    got = oracle.unpack_nibbles(np.array([[0x21, 0xF0, 0x0F]], dtype=np.uint8))
    assert got.tolist() == [[1, 2, 0, 15, 15, 0]]


def _nvfp4_fixture():
    # One expert, 2 rows x 64 columns.  Row 0: every byte 0x53 -> even
    # elements code 3 (1.5), odd elements code 5 (3.0).  Block scales per 16
    # columns: 0x38 (1.0), 0x40 (2.0), 0x30 (0.5), 0xB8 (-1.0).  Row 1: every
    # byte 0xF9 -> even code 9 (-0.5), odd code 15 (-6.0); scales 0x01 (2**-9),
    # 0x7E (448), 0x3C (1.5), 0x00 (0).  Tensor scale 0.25.
    codes = np.empty((1, 2, 32), dtype=np.uint8)
    codes[0, 0] = 0x53
    codes[0, 1] = 0xF9
    scales = np.array([[[0x38, 0x40, 0x30, 0xB8], [0x01, 0x7E, 0x3C, 0x00]]], dtype=np.uint8)
    return {"fmt": 1, "codes": codes, "scales": scales, "zeros": None,
            "tensor_scale": np.array([0.25], dtype=np.float32)}


def test_dequant_nvfp4_hand_values():
    w = oracle.dequant_matrix(_nvfp4_fixture(), 0)
    assert w.shape == (2, 64)
    blk0 = [1.0, 2.0, 0.5, -1.0]
    blk1 = [2.0 ** -9, 448.0, 1.5, 0.0]
    for c in range(64):
        even = c % 2 == 0
        assert w[0, c] == 0.25 * blk0[c // 16] * (1.5 if even else 3.0)
        assert w[1, c] == 0.25 * blk1[c // 16] * (-0.5 if even else -6.0)
    assert w[0, 15] == 0.75 and w[0, 16] == 0.75 and w[0, 17] == 1.5 and w[0, 63] == -0.75
    assert w[1, 16] == -56.0 and w[1, 17] == -672.0


def test_dequant_int4_hand_values():
    # 1 expert, 1 row x 128 columns: byte i holds (i % 16) | ((15 - i % 16) << 4).
    # Group 0: scale 0.5 (fp16 0x3800), zero 8; group 1: scale 1.0 (0x3C00), zero 0.
    codes = np.array([[[(i % 16) | ((15 - i % 16) << 4) for i in range(64)]]], dtype=np.uint8)
    mat = {"fmt": 2, "codes": codes,
           "scales": np.array([[[0x3800, 0x3C00]]], dtype=np.uint16),
           "zeros": np.array([[[8, 0]]], dtype=np.uint8), "tensor_scale": None}
    w = oracle.dequant_matrix(mat, 0)
    for c in range(128):
        i = c // 2
        q = (i % 16) if c % 2 == 0 else 15 - (i % 16)
        expect = 0.5 * (q - 8) if c < 64 else float(q)
        assert w[0, c] == expect, c
    assert w[0, 0] == -4.0 and w[0, 1] == 3.5 and w[0, 63] == -4.0 and w[0, 64] == 0.0


def test_dequant_f32_is_one_rounding_of_exact_product():
    # A tensor scale that is not a power of two: the fp32 weight must be the
    # float32 product of the (exact) block value and the scale, as one IEEE
    # float32 multiply computes it.
    rng = np.random.default_rng(1)
    E, rows, cols = 3, 4, 256
    codes = rng.integers(0, 256, size=(E, rows, cols // 2), dtype=np.uint8)
    scales = rng.integers(0, 256, size=(E, rows, cols // 16), dtype=np.uint8)
    scales[(scales & 0x7F) == 0x7F] = 0x38                           # no NaN codes
    ts = np.array([1.0, 2.0 ** -7, 0.0071234], dtype=np.float32)
    mat = {"fmt": 1, "codes": codes, "scales": scales, "zeros": None, "tensor_scale": ts}
    for e in range(E):
        got = oracle.dequant_matrix_f32(mat, e)
        q = torch.tensor(F.e2m1_value(F.unpack_nibbles(codes[e])), dtype=torch.float32)
        b = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).float()[torch.from_numpy(scales[e].astype(np.int64))]
        ref = (b.repeat_interleave(16, dim=1) * q) * torch.tensor(ts[e])
        assert np.array_equal(got, ref.numpy())


def test_dequant_int4_scale_bias_hand_values():
    # 1 expert, 2 rows x 128 columns; every byte holds codes (c % 16, 15 - c % 16).
    # Row 0: group 0 scale 0.5, bias -1.25; group 1 scale 2.0, bias 3.0.
    # Row 1: group 0 scale -0.25, bias 0; group 1 scale 0 (bias only), bias -7.5.
    codes = np.array([[[(i % 16) | ((15 - i % 16) << 4) for i in range(64)]] * 2], dtype=np.uint8)
    h = lambda v: np.array(v, dtype=np.float16).view(np.uint16)
    mat = {"fmt": 3, "codes": codes, "scales": h([[[0.5, 2.0], [-0.25, 0.0]]]),
           "biases": h([[[-1.25, 3.0], [0.0, -7.5]]]), "zeros": None, "tensor_scale": None}
    w = oracle.dequant_matrix(mat, 0)
    for c in range(128):
        i = c // 2
        q = (i % 16) if c % 2 == 0 else 15 - (i % 16)
        assert w[0, c] == (0.5 * q - 1.25 if c < 64 else 2.0 * q + 3.0), c
        assert w[1, c] == (-0.25 * q if c < 64 else -7.5), c
    # spot values: code 0 gives the bias, code 15 the top of the group's range
    assert w[0, 0] == -1.25 and w[0, 1] == 6.25 and w[0, 64] == 3.0 and w[0, 65] == 33.0


def test_dequant_int4_scale_bias_reduces_to_zero_point():
    # With bias = -scale * z (exact: power-of-two scales) the scale+bias form equals the
    # zero-point form element for element.
    rng = np.random.default_rng(5)
    E, rows, cols = 2, 8, 256
    codes = rng.integers(0, 256, size=(E, rows, cols // 2), dtype=np.uint8)
    zeros = rng.integers(0, 16, size=(E, rows, cols // 64), dtype=np.uint8)
    s = np.exp2(rng.integers(-12, 4, size=zeros.shape)).astype(np.float16)
    s[0, 0, 0] = -s[0, 0, 0]
    b = (-(s.astype(np.float64) * zeros)).astype(np.float16)
    assert np.array_equal(b.astype(np.float64), -(s.astype(np.float64) * zeros))   # the biases are exact
    zp = {"fmt": 2, "codes": codes, "scales": s.view(np.uint16), "zeros": zeros, "tensor_scale": None}
    sb = {"fmt": 3, "codes": codes, "scales": s.view(np.uint16), "biases": b.view(np.uint16), "zeros": None,
          "tensor_scale": None}
    for e in range(E):
        assert np.array_equal(oracle.dequant_matrix(sb, e), oracle.dequant_matrix(zp, e))


def test_dequant_int4_scale_bias_f32_is_one_rounding():
    # fp16 scale * q + fp16 bias is exact in float64; the fp32 weight is its single rounding,
    # which one float32 fused multiply-add also gives.  Scales and biases of very different
    # magnitudes (up to 65504 against fp16 subnormals) make the sum inexact in float32.
    rng = np.random.default_rng(6)
    E, rows, cols = 1, 16, 512
    codes = rng.integers(0, 256, size=(E, rows, cols // 2), dtype=np.uint8)
    mag = np.exp2(rng.uniform(-24, 15.9, size=(E, rows, cols // 64)))
    s = (mag * rng.choice([-1.0, 1.0], size=mag.shape)).astype(np.float16)
    b = (np.exp2(rng.uniform(-24, 15.9, size=mag.shape)) * rng.choice([-1.0, 1.0], size=mag.shape)).astype(np.float16)
    mat = {"fmt": 3, "codes": codes, "scales": s.view(np.uint16), "biases": b.view(np.uint16), "zeros": None,
           "tensor_scale": None}
    got = oracle.dequant_matrix_f32(mat, 0)
    q = F.unpack_nibbles(codes[0]).astype(np.float64)
    exact = np.repeat(s[0].astype(np.float64), 64, axis=1) * q + np.repeat(b[0].astype(np.float64), 64, axis=1)
    # torch's float64 -> float32 conversion (one rounding, nearest even) of the exact value
    ref = torch.from_numpy(exact).to(torch.float32).numpy()
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
    assert np.any(ref.astype(np.float64) != exact)      # some sums really round


def test_dequant_bf16_weights_are_the_bit_patterns():
    # BF16 weights: the codes are bf16 bit patterns; the dequantised matrix is their value,
    # as torch's bfloat16 -> float64 conversion gives it (all 65536 patterns, NaN excepted)
    bits = np.arange(65536, dtype=np.uint16).reshape(1, 256, 256)
    mat = {"fmt": 4, "codes": bits, "scales": None, "zeros": None, "tensor_scale": None}
    w = oracle.dequant_matrix(mat, 0)
    ref = torch.from_numpy(bits[0].astype(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    ok = ~np.isnan(ref)
    assert np.array_equal(w[ok], ref[ok]) and np.array_equal(np.isnan(w), np.isnan(ref))
    # a row subset
    assert np.array_equal(oracle.dequant_matrix(mat, 0, [3, 1]), w[[3, 1]])
