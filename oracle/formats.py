"""Bit-level number formats and exact dequantisation, in float64.

Test infrastructure only (see the package docstring).

The pages name the formats but print no layouts: "[Model] Add Flint
(RecursiveSI/flint)" (section "What happened") serves NVFP4 weights
weight-only as W4A16, and "Recursive Flint: 125 tok/s on an M4 Pro,
measured where it matters least" (table in "What actually shipped") lists
a group-64 affine INT4 build.  The readings taken here:

* e2m1 (the NVFP4 element): sign bit, 2 exponent bits (bias 1), 1 mantissa
  bit; exponent 0 is subnormal.  Values +-{0, 0.5, 1, 1.5, 2, 3, 4, 6}.
* e4m3 "FN" (the NVFP4 block scale): sign bit, 4 exponent bits (bias 7),
  3 mantissa bits; exponent 0 is subnormal; S.1111.111 is NaN (invalid
  input); there are no infinities.  Largest value 448.
* NVFP4 weight = fp32 tensor scale * e4m3 block scale (one per 16
  consecutive elements along the reduction axis) * e2m1 code.
* INT4 group-64 affine weight = fp16 scale * (q - z), q and z in 0..15,
  one (scale, zero) per 64 consecutive elements along the reduction axis.
* The other reading of "affine" (scale and bias, as MLX stores its affine
  4-bit groups): weight = fp16 scale * q + fp16 bias, q in 0..15, one
  (scale, bias) per 64 consecutive elements along the reduction axis.  The
  zero-point form is the special case bias = -scale * z.
* BF16 weights (the 16-bit checkpoint that "[Model] Add Flint
  (RecursiveSI/flint)", section "What happened", serves beside NVFP4):
  ``codes`` holds the bf16 bit patterns [E, rows, cols] themselves.
* A matrix is stored row-major as [out, in]; element 2i of a row sits in
  the low nibble of byte i, element 2i+1 in the high nibble.

A matrix is a dict: ``fmt`` (1 = NVFP4, 2 = INT4 group 64), ``codes``
uint8 [E, rows, cols/2], ``scales`` (NVFP4: uint8 e4m3 codes
[E, rows, cols/16]; INT4: uint16 fp16 bit patterns [E, rows, cols/64]),
``zeros`` (INT4: uint8 [E, rows, cols/64]; else None), ``tensor_scale``
(NVFP4: float32 [E]; else None), ``biases`` (INT4 scale + bias: uint16 fp16
bit patterns [E, rows, cols/64]; else absent or None).
"""

import numpy as np

FMT_NVFP4 = 1
FMT_INT4_G64 = 2
FMT_INT4_SB = 3
FMT_BF16 = 4
NVFP4_BLOCK = 16
INT4_GROUP = 64


def bf16_bits_to_f64(bits):
    """bfloat16 bit patterns -> float64 (exact): the float32 whose high half is the pattern."""
    b = np.asarray(bits).astype(np.uint32)
    return (b << 16).view(np.float32).astype(np.float64)


def fp16_bits_to_f64(bits):
    """IEEE binary16 bit patterns -> float64 (exact)."""
    return np.asarray(bits).astype(np.uint16).view(np.float16).astype(np.float64)


def e2m1_value(nib):
    """Value of a 4-bit e2m1 code (0..15) from its bit fields."""
    n = np.asarray(nib).astype(np.int64)
    s = (n >> 3) & 1
    e = (n >> 1) & 3
    m = n & 1
    mag = np.where(e == 0, 0.5 * m, (1.0 + 0.5 * m) * np.exp2(e - 1.0))
    return np.where(s == 1, -mag, mag)


def e4m3fn_value(byte):
    """Value of an 8-bit e4m3 FN code from its bit fields; NaN for S.1111.111."""
    b = np.asarray(byte).astype(np.int64)
    s = (b >> 7) & 1
    e = (b >> 3) & 15
    m = b & 7
    mag = np.where(e == 0, (m / 8.0) * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return np.where(s == 1, -mag, mag)


def unpack_nibbles(codes):
    """uint8 [..., n/2] -> int64 [..., n]; element 2i = low nibble of byte i."""
    c = np.asarray(codes).astype(np.int64)
    out = np.empty(c.shape[:-1] + (2 * c.shape[-1],), dtype=np.int64)
    out[..., 0::2] = c & 15
    out[..., 1::2] = c >> 4
    return out


def _rows(a, rows):
    a = np.asarray(a)
    return a if rows is None else a[np.asarray(rows)]


def dequant_matrix(mat, expert, rows=None):
    """Exact float64 weights [rows, cols] of one expert of a packed matrix
    (only the listed rows when ``rows`` is given)."""
    sub = dict(mat)
    for key in ("codes", "scales", "zeros", "biases"):
        if mat.get(key) is not None:
            sub[key] = {expert: _rows(mat[key][expert], rows)}
    mat = sub
    if mat["fmt"] == FMT_BF16:
        return bf16_bits_to_f64(mat["codes"][expert])
    q = unpack_nibbles(mat["codes"][expert])
    rows, cols = q.shape
    if mat["fmt"] == FMT_NVFP4:
        blk = e4m3fn_value(mat["scales"][expert])            # [rows, cols/16]
        assert blk.shape == (rows, cols // NVFP4_BLOCK)
        ts = float(np.float32(mat["tensor_scale"][expert]))
        return ts * (np.repeat(blk, NVFP4_BLOCK, axis=1) * e2m1_value(q))
    if mat["fmt"] == FMT_INT4_G64:
        s = fp16_bits_to_f64(mat["scales"][expert])          # [rows, cols/64]
        z = np.asarray(mat["zeros"][expert]).astype(np.float64)
        assert s.shape == (rows, cols // INT4_GROUP) and z.shape == s.shape
        return np.repeat(s, INT4_GROUP, axis=1) * (q - np.repeat(z, INT4_GROUP, axis=1))
    if mat["fmt"] == FMT_INT4_SB:
        # s*q has at most 15 significant bits and s*q + b spans at most 45 bits
        # (fp16 magnitudes 2**-24 .. 2**20): exact in float64
        s = fp16_bits_to_f64(mat["scales"][expert])          # [rows, cols/64]
        b = fp16_bits_to_f64(mat["biases"][expert])
        assert s.shape == (rows, cols // INT4_GROUP) and b.shape == s.shape
        return np.repeat(s, INT4_GROUP, axis=1) * q + np.repeat(b, INT4_GROUP, axis=1)
    raise ValueError("unknown weight format %r" % (mat["fmt"],))


def dequant_matrix_f32(mat, expert):
    """The exact weights rounded once (to nearest, ties to even) to float32.

    For NVFP4, block scale * code has at most 6 significant bits, so the
    float64 product with the fp32 tensor scale is exact and this is a single
    rounding of the true value (bf16 weights are exact).  INT4 zero-point weights (at most 15
    significant bits) are exact in float32; scale + bias weights are exact in
    float64, so this is again one rounding of the true value.
    """
    return dequant_matrix(mat, expert).astype(np.float32)


def rne_bf16(x):
    """Round float64 values directly to bfloat16 (nearest, ties to even).

    Rounds once from float64 (not through float32, which would round twice).
    bfloat16 keeps 8 significant bits, the float32 exponent range, and
    subnormals down to 2**-133.  Returns float64 values that bfloat16 holds.
    """
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)                       # x = m * 2**e, 0.5 <= |m| < 1
    q = np.maximum(e - 8, -133)              # exponent of one unit in the last place
    y = np.ldexp(np.rint(np.ldexp(x, -q)), q)
    big = (2.0 - 2.0 ** -7) * 2.0 ** 127
    return np.where(np.abs(y) > big, np.copysign(np.inf, x), y)


def f64_to_bf16_bits(x):
    """bfloat16 bit patterns (uint16) of values that bfloat16 holds exactly."""
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    return (f.view(np.uint32) >> 16).astype(np.uint16)
