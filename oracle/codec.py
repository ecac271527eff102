"""NVFP4 codec, oracle side (test infrastructure; see the package docstring).

Formats, as the pages define them:

* an element is a 4-bit E2M1 float, two elements per byte, and each block of
  16 consecutive elements carries one 8-bit E4M3 scale: 64 data bits plus 8
  scale bits, 4.5 bits per value ("NVFP4 KV cache prefill vs decode
  performance", section "NVFP4 stores 4.5 bits per value before padding";
  "NVFP4 KV cache vs NVFP4 weights", section "NVFP4 KV cache vs NVFP4
  weights");
* a second, per-tensor scale ``g`` brings the tensor into the range that
  E2M1 codes under E4M3 block scales can cover (same page and section).

Readings where the pages are silent (each is listed in the design notes):

* E2M1 is sign-magnitude with a 2-bit exponent of bias 1 and a 1-bit
  mantissa; bit 3 is the sign.  Magnitude codes 0..7 are the values
  0, 0.5, 1, 1.5, 2, 3, 4, 6.
* E4M3 is the OCP "FN" variant: bias 7, subnormals, no infinities, 0x7F is
  NaN, largest finite value 448 (code 0x7E).  Block scales are non-negative.
* The block scale is ``s = E4M3(fl32(amax / 6))`` where ``amax`` is the
  largest magnitude in the block after division by ``g`` and ``fl32`` is
  IEEE float32 division.  For bf16 inputs and ``g = 1`` this equals E4M3
  rounding of the exact quotient: with ``amax = k 2^e`` and k < 256, the
  quotient is exact in float32 when 3 divides k, and otherwise lies at a
  relative distance of at least about 2^-9 from every E4M3 rounding boundary,
  far beyond the 2^-24 that float32 rounding can move it.
* Both roundings are round-to-nearest with ties to the even code, and
  saturate at the largest finite value.
* The element code is ``sign(y) << 3 | RNE_sat(|y| / s)``; the sign bit
  always copies the sign bit of ``y`` (so -0 and small negatives give 0x8),
  and a zero scale gives magnitude 0 for every element of the block.
* Nibble order: element 2i is the low nibble of byte i, element 2i+1 the
  high nibble.
"""
from __future__ import annotations

import numpy as np

BLOCK = 16          # elements per scale block
E2M1_MAX = 6.0      # largest E2M1 magnitude
E4M3_MAX_CODE = 0x7E


def e2m1_value(code) -> np.ndarray:
    """Value of a 4-bit E2M1 code (0..15), from its sign, exponent and mantissa bits."""
    code = np.asarray(code).astype(np.int64)
    e = (code >> 1) & 3
    m = (code & 1).astype(np.float64)
    mag = np.where(e == 0, m * 0.5, np.ldexp(1.0 + m / 2.0, (e - 1).astype(np.int64)))
    return np.where((code >> 3) & 1, -mag, mag)


def e4m3_value(code) -> np.ndarray:
    """Value of an 8-bit E4M3FN code (bias 7; subnormal when the exponent field is 0)."""
    code = np.asarray(code).astype(np.int64)
    e = (code >> 3) & 15
    m = (code & 7).astype(np.float64)
    mag = np.where(e == 0, np.ldexp(m / 8.0, -6), np.ldexp(1.0 + m / 8.0, (e - 7).astype(np.int64)))
    mag = np.where((code & 0x7F) == 0x7F, np.nan, mag)
    return np.where((code >> 7) & 1, -mag, mag)


# Non-negative finite grids in code order (both formats are monotone in their codes).
_E2M1_POS = e2m1_value(np.arange(8))
_E4M3_POS = e4m3_value(np.arange(E4M3_MAX_CODE + 1))


def _nearest_even(v: np.ndarray, grid: np.ndarray) -> np.ndarray:
    """Index of the grid value nearest to each v >= 0; ties go to the even index.

    Values above the last grid point map to the last index (saturation).
    Distances are exact in float64 for the operands used here (see module doc).
    """
    v = np.asarray(v, dtype=np.float64)
    top = len(grid) - 1
    hi = np.searchsorted(grid, v, side="left").clip(0, top)
    lo = (hi - 1).clip(0, top)
    d_lo = v - grid[lo]
    d_hi = grid[hi] - v
    take_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    return np.where(take_hi, hi, lo)


def e4m3_encode(v) -> np.ndarray:
    """E4M3FN code of a non-negative value: round to nearest, ties to even, saturate at 448."""
    return _nearest_even(v, _E4M3_POS).astype(np.uint8)


def e2m1_encode(y, s) -> np.ndarray:
    """E2M1 code of y under block scale s (> 0 or 0), as a uint8 in 0..15."""
    y = np.asarray(y, dtype=np.float64)
    s = np.broadcast_to(np.asarray(s, dtype=np.float64), y.shape)
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.abs(y) / s
    mag = np.where(s > 0, _nearest_even(np.where(s > 0, r, 0.0), _E2M1_POS), 0)
    sign = np.signbit(y).astype(np.int64) << 3
    return (sign | mag).astype(np.uint8)


def block_scale_codes(y: np.ndarray) -> np.ndarray:
    """Scale code of every 16-value block along the last axis of float32 values y."""
    yb = np.asarray(y, dtype=np.float32).reshape(*y.shape[:-1], y.shape[-1] // BLOCK, BLOCK)
    amax = np.abs(yb).max(axis=-1)
    quotient = (amax / np.float32(E2M1_MAX)).astype(np.float32)  # IEEE float32 division
    return e4m3_encode(quotient.astype(np.float64))


def quantize(x: np.ndarray, g: float = 1.0):
    """Quantize float32 values along the last axis (a multiple of 16 long).

    Returns (element codes uint8 [..., D], scale codes uint8 [..., D/16]).
    ``y = fl32(x / g)``; the scale and element codes follow the module doc.
    """
    x = np.asarray(x, dtype=np.float32)
    y = (x / np.float32(g)).astype(np.float32)
    sc = block_scale_codes(y)
    s = e4m3_value(sc)
    sb = np.repeat(s, BLOCK, axis=-1)
    codes = e2m1_encode(y.astype(np.float64), sb)
    return codes, sc


# ---- FP8 (E4M3FN) KV cache, the control format --------------------------------------------
# Every value is one E4M3FN byte under a per-tensor scale g: the writer stores
# E4M3_RNE_sat(fl32(x / g)) with the sign bit copied from y, the reader multiplies by g.  (The
# pages compare NVFP4 against an FP8 cache throughout; its exact layout is a reading.)

def e4m3_encode_signed(y) -> np.ndarray:
    """E4M3FN code of float values: sign bit 7 copied from y, magnitude rounded to nearest with
    ties to the even code, saturating at 448 (0x7E)."""
    y = np.asarray(y, dtype=np.float64)
    return ((np.signbit(y).astype(np.uint8) << 7) | e4m3_encode(np.abs(y))).astype(np.uint8)


def quantize_fp8(x: np.ndarray, g: float = 1.0) -> np.ndarray:
    """FP8 cache codes of float32 values: E4M3FN of y = fl32(x / g)."""
    x = np.asarray(x, dtype=np.float32)
    y = (x / np.float32(g)).astype(np.float32)
    return e4m3_encode_signed(y.astype(np.float64))


def dequantize_fp8(codes: np.ndarray, g: float = 1.0) -> np.ndarray:
    """Read-side value of FP8 cache codes: g * e4m3(code), in float64."""
    return float(g) * e4m3_value(np.asarray(codes, dtype=np.uint8))


def pack(codes: np.ndarray) -> np.ndarray:
    """Two E2M1 codes per byte: element 2i in the low nibble, 2i+1 in the high nibble."""
    codes = np.asarray(codes, dtype=np.uint8)
    return (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)


def unpack(packed: np.ndarray) -> np.ndarray:
    packed = np.asarray(packed, dtype=np.uint8)
    out = np.empty(packed.shape[:-1] + (packed.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = packed & 0xF
    out[..., 1::2] = packed >> 4
    return out


def dequantize(packed: np.ndarray, scale_codes: np.ndarray, g: float = 1.0) -> np.ndarray:
    """Read-side value of every element: g * s * e2m1(code), in float64."""
    codes = unpack(packed)
    s = np.repeat(e4m3_value(scale_codes), BLOCK, axis=-1)
    return float(g) * s * e2m1_value(codes)


def fp16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact value of IEEE binary16 bit patterns, as float32 (every binary16 value is one)."""
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float32)


def input_to_f32(bits: np.ndarray, input_dtype: str = "bf16") -> np.ndarray:
    """Writer input bit patterns (bf16 or fp16) -> their exact float32 values."""
    if input_dtype == "bf16":
        return bf16_to_f32(bits)
    if input_dtype == "fp16":
        return fp16_to_f32(bits)
    raise ValueError(f"input dtype {input_dtype!r}")


def round_to_dtype(x: np.ndarray, out_dtype: str) -> np.ndarray:
    """float32 values rounded to nearest-even in bf16 / fp16 (as bit patterns), or kept as
    float32: the output types of the standalone dequantization."""
    x = np.asarray(x, dtype=np.float32)
    if out_dtype == "f32":
        return x
    if out_dtype == "fp16":
        return x.astype(np.float16).view(np.uint16)
    if out_dtype == "bf16":
        b = x.view(np.uint32).astype(np.uint64)
        r = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
        return r.astype(np.uint16)
    raise ValueError(f"output dtype {out_dtype!r}")


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact value of bfloat16 bit patterns, as float32."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)
