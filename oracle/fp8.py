"""OCP FP8 E4M3 ("finite-only, max 448") decoding, written from the format definition.

Cites: *Module 10: Inference and Deployment Serving* (wrwei.github.io), the
number-formats discussion under "Range and resolution answer different
questions": E4M3 variants differ in how they treat infinity and NaN, and the
page's format table uses the finite-only convention whose largest value is 448.
*The Mathematics of Transformer Inference* (hs-black), §11: an 8-bit KV cache
halves KV bytes, and dequantisation is fused into the kernel.

The bit layout (sign | 4-bit exponent, bias 7 | 3-bit mantissa) and the
subnormal rule come from the OCP 8-bit floating point specification:
  exponent field 0      -> (-1)^s * (m / 8) * 2^-6          (zero and subnormals)
  exponent 1..15        -> (-1)^s * (1 + m / 8) * 2^(e - 7)
  exponent 15, m = 7    -> NaN (0x7F, 0xFF); there is no infinity.
So the largest finite value is (1 + 6/8) * 2^8 = 448, as the page states.

Encoding (used by the quantised append) is the inverse written as a search:
the nearest finite value, a tie going to the code whose mantissa is even (round
to nearest even), magnitudes beyond 448 saturating to 448, the sign kept (so
-0.0 gives 0x80).  *The Mathematics of Transformer Inference* §11: quantising is
x ~ s * round(x / s).
"""
import numpy as np


def decode_e4m3fn(codes: np.ndarray) -> np.ndarray:
    """uint8 E4M3 codes -> float64 values (NaN for the two NaN codes)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where((c >> 7) & 1, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    subnormal = sign * (m / 8.0) * 2.0 ** -6
    normal = sign * (1.0 + m / 8.0) * np.power(2.0, (e - 7).astype(np.float64))
    out = np.where(e == 0, subnormal, normal)
    out = np.where((e == 0xF) & (m == 7), np.nan, out)
    return out


FP8_MAX = 448.0


def _positive_values():
    """Codes 0x00..0x7E (every non-negative finite value) and their values, ascending."""
    codes = np.arange(0x7F, dtype=np.uint8)
    return codes, decode_e4m3fn(codes)


def encode_e4m3fn(x: np.ndarray) -> np.ndarray:
    """float -> E4M3 codes (uint8): nearest finite value, ties to the even code,
    saturating at +-448; NaN -> 0x7F (with its sign bit)."""
    x = np.asarray(x, dtype=np.float64)
    codes, vals = _positive_values()
    a = np.minimum(np.abs(x), FP8_MAX)
    i = np.clip(np.searchsorted(vals, a, side="left"), 1, len(vals) - 1)
    below, above = vals[i - 1], vals[i]
    d_below, d_above = a - below, above - a
    take_above = (d_above < d_below) | ((d_above == d_below) & (codes[i] % 2 == 0))
    mag = np.where(take_above, codes[i], codes[i - 1]).astype(np.int64)
    mag = np.where(np.isnan(x), 0x7F, mag)
    return (mag | (np.signbit(x).astype(np.int64) << 7)).astype(np.uint8)
