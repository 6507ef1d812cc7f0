"""KV-cache number formats, written from their definitions (oracle side).

The pages name the formats only: FP16/BF16 caches and an 8-bit floating-point
KV cache that halves the bytes of FP16 (vLLM V1 article, "FP8 KV cache
quantization"; itwiki "vLLM", "Engine structure and main features":
``--kv-cache-dtype auto/fp8``).  The 8-bit format read here is OCP E4M3FN:
1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits, subnormals at
exponent field 0, no infinities, NaN only at S.1111.111, largest finite 448.

Encoding is round-to-nearest, ties to even, done by scaling to the format's
quantum in float64 (exact for these widths) and rounding with ``np.rint``.
The 8-bit encoder saturates finite overflow (and infinities) to +-448 and
keeps NaN as NaN; this saturation is a reading of the pages, which are
silent on overflow.  NaN inputs become the canonical quiet NaN of the target
with the sign kept.
"""

from __future__ import annotations

import numpy as np

# ---------------------------------------------------------------------------
# decoding to float64
# ---------------------------------------------------------------------------

def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> float64 (a bf16 is the top half of an fp32)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def f16_to_f64(bits: np.ndarray) -> np.ndarray:
    """float16 values, or their uint16 bit patterns -> float64."""
    a = np.asarray(bits)
    if a.dtype != np.float16:
        a = a.astype(np.uint16, copy=False).view(np.float16)
    return a.astype(np.float64)


def f32_to_f64(x: np.ndarray) -> np.ndarray:
    a = np.asarray(x)
    if a.dtype == np.uint32:
        a = a.view(np.float32)
    return a.astype(np.float64)


def e4m3fn_table() -> np.ndarray:
    """The 256 values of OCP E4M3FN, indexed by code, in float64."""
    out = np.empty(256, dtype=np.float64)
    for code in range(256):
        sign = -1.0 if code & 0x80 else 1.0
        e = (code >> 3) & 0xF
        m = code & 0x7
        if e == 0xF and m == 0x7:
            out[code] = np.nan
        elif e == 0:
            out[code] = sign * (m / 8.0) * 2.0 ** (1 - 7)
        else:
            out[code] = sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return out


_E4M3 = e4m3fn_table()


def e4m3fn_to_f64(codes: np.ndarray) -> np.ndarray:
    return _E4M3[np.asarray(codes, dtype=np.uint8)]


def decode(raw: np.ndarray, dtype: str) -> np.ndarray:
    """Raw storage bits (or float32 values) of ``dtype`` -> float64."""
    if dtype == "f32":
        return f32_to_f64(raw)
    if dtype == "f16":
        return f16_to_f64(raw)
    if dtype == "bf16":
        return bf16_to_f64(raw)
    if dtype == "fp8_e4m3":
        return e4m3fn_to_f64(raw)
    raise ValueError(dtype)


def to_f32(raw: np.ndarray, dtype: str) -> np.ndarray:
    """Source K/V (f32 values, f16 values or bf16 bits) -> float32, exactly."""
    if dtype == "f32":
        return np.asarray(raw, dtype=np.float32)
    if dtype == "f16":
        a = np.asarray(raw)
        if a.dtype != np.float16:
            a = a.astype(np.uint16, copy=False).view(np.float16)
        return a.astype(np.float32)
    if dtype == "bf16":
        return (np.asarray(raw, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)
    raise ValueError(dtype)


# ---------------------------------------------------------------------------
# encoding (round to nearest, ties to even)
# ---------------------------------------------------------------------------

def _round_to_format(x: np.ndarray, mant_bits: int, emin: int) -> np.ndarray:
    """Round finite float64 magnitudes to a binary format with ``mant_bits``
    stored mantissa bits and smallest normal exponent ``emin``; unbounded
    exponent range above.  Ties go to the even quantum multiple."""
    a = np.abs(x)
    with np.errstate(divide="ignore"):
        _, e2 = np.frexp(a)          # a = f * 2**e2, f in [0.5, 1)
    e = np.maximum(e2.astype(np.int64) - 1, emin)   # exponent of the leading bit
    e = np.where(a == 0, emin, e)
    quantum = np.ldexp(1.0, (e - mant_bits).astype(np.int32))
    q = np.rint(a / quantum)          # exact division by a power of two
    return np.copysign(q * quantum, x)


def f32_to_bf16(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bits, RNE; overflow to inf; NaN -> sign|0x7FC0."""
    x = np.asarray(x, dtype=np.float32)
    xd = x.astype(np.float64)
    fin = np.isfinite(xd)
    r = np.where(fin, _round_to_format(np.where(fin, xd, 0.0), 7, -126), xd)
    # a rounded magnitude at or above 2**128 is past the largest finite bf16
    r = np.where(np.abs(r) >= 2.0 ** 128, np.copysign(np.inf, xd), r)
    with np.errstate(over="ignore"):
        bits = (r.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    nan = np.isnan(xd)
    sign = (x.view(np.uint32) >> 16).astype(np.uint16) & np.uint16(0x8000)
    return np.where(nan, sign | np.uint16(0x7FC0), bits).astype(np.uint16)


def f32_to_f16(x: np.ndarray) -> np.ndarray:
    """float32 -> float16 bits, RNE; overflow to inf; NaN -> sign|0x7E00."""
    x = np.asarray(x, dtype=np.float32)
    xd = x.astype(np.float64)
    fin = np.isfinite(xd)
    r = np.where(fin, _round_to_format(np.where(fin, xd, 0.0), 10, -14), xd)
    r = np.where(np.abs(r) > 65504.0, np.copysign(np.inf, xd), r)
    bits = r.astype(np.float16).view(np.uint16)   # r is exactly representable (or inf)
    nan = np.isnan(xd)
    sign = (x.view(np.uint32) >> 16).astype(np.uint16) & np.uint16(0x8000)
    return np.where(nan, sign | np.uint16(0x7E00), bits).astype(np.uint16)


# the 127 non-negative finite codes 0x00..0x7E have increasing values
_E4M3_POS = _E4M3[:0x7F]


def f64_to_e4m3fn(y: np.ndarray) -> np.ndarray:
    """float64 -> E4M3FN codes: RNE, saturate to +-448, NaN -> sign|0x7F."""
    y = np.asarray(y, dtype=np.float64)
    nan = np.isnan(y)
    yy = np.where(nan, 0.0, y)
    r = _round_to_format(np.clip(yy, -448.0, 448.0), 3, -6)
    r = np.clip(r, -448.0, 448.0)          # a tie above 448 rounds to 512: saturate
    mag = np.searchsorted(_E4M3_POS, np.abs(r))   # r is a format value: exact hit
    codes = mag.astype(np.uint8) | np.where(np.signbit(yy), 0x80, 0).astype(np.uint8)
    nan_code = np.where(np.signbit(y), 0xFF, 0x7F).astype(np.uint8)
    return np.where(nan, nan_code, codes).astype(np.uint8)


def f32_to_e4m3fn_scaled(x: np.ndarray, scale: float) -> np.ndarray:
    """Quantise fp32 values with a per-tensor scale: code = e4m3(fl32(x / scale)).

    The division is the correctly rounded float32 quotient (NumPy float32
    division is IEEE), then rounded to E4M3FN as above.
    """
    x = np.asarray(x, dtype=np.float32)
    with np.errstate(over="ignore", invalid="ignore", divide="ignore"):
        y = x / np.float32(scale)
    return f64_to_e4m3fn(y.astype(np.float64))


def encode(x_f32: np.ndarray, dtype: str, scale: float = 1.0) -> np.ndarray:
    """float32 values -> storage bits of ``dtype`` (the cache write's enc)."""
    if dtype == "f32":
        return np.asarray(x_f32, dtype=np.float32).view(np.uint32)
    if dtype == "bf16":
        return f32_to_bf16(x_f32)
    if dtype == "f16":
        return f32_to_f16(x_f32)
    if dtype == "fp8_e4m3":
        return f32_to_e4m3fn_scaled(x_f32, scale)
    raise ValueError(dtype)
