"""Number formats used by the attention path, written from their definitions.

* bfloat16: 1 sign, 8 exponent (bias 127), 7 fraction bits; 8 significant
  bits. Round-to-nearest-even.
* OCP FP8 E4M3FN ("e4m3"): 1 sign, 4 exponent (bias 7), 3 fraction bits;
  exponent field 0 holds subnormals m/8 * 2^-6; all-ones exponent with all-ones
  fraction (0x7F / 0xFF) is NaN; there is no infinity; the largest finite
  magnitude is 1.75 * 2^8 = 448 (OCP 8-bit Floating Point Specification, E4M3
  encoding table). The pages only say that FP8 attention variants exist
  (Japanese summary, third paragraph; "Key takeaways" of the English card);
  the format is this library's reading.

Rounding is done on exact float64 values: for a value whose exponent is e
(2^e <= |x| < 2^(e+1)), with e clamped below at the format's minimum normal
exponent, the representable neighbours are multiples of 2^(e - fraction_bits);
dividing by that power of two is exact, ``np.rint`` rounds half to even, and
multiplying back is exact.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
E4M3_EMIN = -6          # exponent of the smallest normal, 2^-6
E4M3_FRAC = 3
BF16_EMIN = -126
BF16_FRAC = 7


def _round_to_grid(a: np.ndarray, frac_bits: int, emin: int) -> np.ndarray:
    """RNE of non-negative float64 ``a`` to a binary format with ``frac_bits``
    fraction bits and minimum normal exponent ``emin`` (no overflow handling)."""
    a = np.asarray(a, dtype=np.float64)
    _, x = np.frexp(a)                 # a = f * 2^x, f in [0.5, 1)
    e = np.maximum(x - 1, emin)        # binade exponent, subnormals share emin
    quantum = np.ldexp(1.0, e - frac_bits)
    return np.rint(a / quantum) * quantum


def bf16_round(x) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 (ties to even); returns float64."""
    x = np.asarray(x, dtype=np.float64)
    r = _round_to_grid(np.abs(x), BF16_FRAC, BF16_EMIN)
    return np.copysign(r, x)


def e4m3_decode(codes) -> np.ndarray:
    """float64 value of each e4m3 byte (NaN for 0x7F and 0xFF)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c >> 7, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    normal = np.ldexp(1.0 + m / 8.0, e - 7)
    sub = np.ldexp(m / 8.0, E4M3_EMIN)
    v = np.where(e == 0, sub, normal)
    v = np.where((e == 15) & (m == 7), np.nan, v)
    return sign * v


def e4m3_encode(x) -> np.ndarray:
    """Round float64 values to e4m3 codes, nearest-even, saturating at +-448.

    NaN maps to 0x7F (sign kept). Negative zero keeps its sign bit."""
    x = np.asarray(x, dtype=np.float64)
    neg = np.signbit(x)
    a = np.abs(x)
    nan = np.isnan(a)
    a = np.where(nan, 0.0, np.minimum(a, E4M3_MAX))
    r = _round_to_grid(a, E4M3_FRAC, E4M3_EMIN)      # representable magnitude
    _, xe = np.frexp(r)
    e = xe - 1
    is_normal = r >= np.ldexp(1.0, E4M3_EMIN)
    frac_normal = np.rint((r / np.ldexp(1.0, np.where(is_normal, e, 0)) - 1.0) * 8.0)
    code_normal = ((e + 7) << 3) + frac_normal.astype(np.int64)
    code_sub = np.rint(r / np.ldexp(1.0, E4M3_EMIN - E4M3_FRAC)).astype(np.int64)
    code = np.where(is_normal, code_normal, code_sub)
    code = np.where(nan, 0x7F, code)
    code = code | np.where(neg, 0x80, 0)
    return code.astype(np.uint8)


def quantize_per_tensor(x):
    """Per-tensor absmax quantisation to e4m3, all arithmetic in fp32.

    s = fp32(448 / max|x|); y = fp32(x * s), clamped to [-448, 448]; codes =
    e4m3 RNE of y; descale = fp32(1 / s). An all-zero tensor (or a maximum so
    small that 448/max overflows fp32) uses s = 1. Returns
    (codes uint8 array, descale float32, s float32)."""
    if hasattr(x, "detach"):
        x = x.detach().to("cpu").float().numpy()
    x = np.asarray(x, dtype=np.float32)
    amax = np.float32(np.max(np.abs(x))) if x.size else np.float32(0.0)
    with np.errstate(divide="ignore", over="ignore"):
        s = np.float32(448.0) / amax if amax > 0 else np.float32(1.0)
    if not np.isfinite(s):
        s = np.float32(1.0)
    y = np.multiply(x, s, dtype=np.float32)
    y = np.clip(y, np.float32(-E4M3_MAX), np.float32(E4M3_MAX))
    codes = e4m3_encode(y.astype(np.float64))
    descale = np.float32(1.0) / s
    return codes, np.float32(descale), np.float32(s)
