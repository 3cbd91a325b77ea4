"""Number formats of the FP8 x FP4 MoE path (oracle side, test infrastructure).

Cited passages (page titles as published):
* "MegaMoE" code walk-through (infra.simphoni.uk), section 7.1 "precision
  configuration": weights in FP4 E2M1, UE8M0 power-of-two scales packed four
  to a 32-bit word.  The page's value list for E2M1 is garbled; the OCP
  Microscaling (MX) v1.0 definition is used: no NaN/Inf, largest value 6.
* Same page, section 7.2 "block scaling": one scale per 32 elements along K.
* DeepGEMM MegaMoE reading notes (notes.kuangjux.top), "numerical formats"
  table: activations FP8 E4M3, L1 epilogue output FP8 E4M3, L2 output BF16.

Readings where the pages are silent: E4M3 is the OCP "FN" flavour (max 448,
one NaN pattern per sign, no infinities); E8M0 code c means 2**(c-127); the
FP4 byte holds the even-K element in its low nibble.

All decoders return float64 values, which represent every code exactly.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
E2M1_MAX = 6.0


def _e4m3_table() -> np.ndarray:
    """Value of every 8-bit E4M3FN code (sign | 4-bit exponent, bias 7 | 3-bit mantissa)."""
    vals = np.empty(256, dtype=np.float64)
    for c in range(256):
        sign = -1.0 if c & 0x80 else 1.0
        e = (c >> 3) & 0xF
        m = c & 0x7
        if e == 0xF and m == 0x7:
            vals[c] = np.nan
        elif e == 0:
            vals[c] = sign * m * 2.0 ** -9          # subnormal: m/8 * 2**(1-7)
        else:
            vals[c] = sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return vals


def _e2m1_table() -> np.ndarray:
    """Value of every 4-bit E2M1 code (sign | 2-bit exponent, bias 1 | 1-bit mantissa)."""
    vals = np.empty(16, dtype=np.float64)
    for c in range(16):
        sign = -1.0 if c & 0x8 else 1.0
        e = (c >> 1) & 0x3
        m = c & 0x1
        if e == 0:
            vals[c] = sign * m * 0.5                # subnormal: m/2 * 2**(1-1)
        else:
            vals[c] = sign * (1.0 + m / 2.0) * 2.0 ** (e - 1)
    return vals


E4M3_TABLE = _e4m3_table()
E2M1_TABLE = _e2m1_table()


def decode_e4m3(codes: np.ndarray) -> np.ndarray:
    return E4M3_TABLE[np.asarray(codes, dtype=np.uint8)]


def decode_e8m0(codes: np.ndarray) -> np.ndarray:
    """UE8M0 scale: 2**(c - 127); code 255 is NaN and never produced."""
    c = np.asarray(codes, dtype=np.int64)
    out = np.ldexp(1.0, c - 127)
    return np.where(c == 255, np.nan, out)


def unpack_fp4(packed: np.ndarray) -> np.ndarray:
    """[..., K/2] bytes -> [..., K] nibble codes, even K index in the low nibble."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = p & 0x0F
    out[..., 1::2] = p >> 4
    return out


def decode_e2m1_packed(packed: np.ndarray) -> np.ndarray:
    return E2M1_TABLE[unpack_fp4(packed)]


def dequant_blocks(values: np.ndarray, scale_codes: np.ndarray, block: int = 32) -> np.ndarray:
    """values [..., K] (float64) times 2**(sf-127) repeated over each run of `block` along K."""
    s = decode_e8m0(scale_codes)
    return values * np.repeat(s, block, axis=-1)


def f32_bits(x: np.ndarray) -> np.ndarray:
    return np.asarray(x, dtype=np.float32).view(np.uint32)


def bf16_rne(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16, nearest-even; returned as float32 values.

    Done on the raw bits: add 0x7FFF plus the lowest kept bit, then drop the
    low 16 bits.  Inputs are finite (NaN never occurs on this path).
    """
    u = f32_bits(x).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return (u.astype(np.uint32) << 16).view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) of float32 values that are already bf16-exact."""
    return (f32_bits(x) >> 16).astype(np.uint16)


def bf16_from_bits(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# Positive E4M3 values in code order 0x00..0x7E (monotone), used for encoding.
_E4M3_POS = E4M3_TABLE[:0x7F]


def encode_e4m3_rne(v: np.ndarray) -> np.ndarray:
    """Round real values (float64, |v| <= 448) to the nearest E4M3 value, ties to even.

    The E4M3 grid has step 2**-9 below 2**-6 (subnormals) and step
    2**(floor(log2|v|) - 3) above.  Rounding is done on that grid with
    numpy's round-half-even, then the result's code is looked up.  The sign
    of zero is kept (-0 -> 0x80).
    """
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    if np.any(a > E4M3_MAX) or np.any(np.isnan(a)):
        raise ValueError("E4M3 encoder input outside the finite range")
    _, e = np.frexp(a)                      # a = f * 2**e, f in [0.5, 1)
    exp = np.maximum(e - 1, -6)             # floor(log2 a), clamped at the subnormal range
    step = np.ldexp(1.0, exp - 3)
    q = np.rint(a / step) * step            # exact: a/step scales by a power of two
    code = np.searchsorted(_E4M3_POS, q).astype(np.uint8)
    assert np.all(_E4M3_POS[code] == q)
    neg = np.signbit(v)
    return np.where(neg, code | 0x80, code).astype(np.uint8)


def requant_scale_code(amax: np.ndarray) -> np.ndarray:
    """UE8M0 code of the FP8 requant scale for a 32-channel group with this amax.

    Reading of the L1-epilogue description (reading notes, "L1 epilogue:
    SwiGLU and requantization"; walk-through section 4.6): the scale is a
    power of two 2**s and values are divided by it to land in FP8 range.  The
    oracle takes the smallest such power with amax / 2**s <= 448, found here
    from frexp and a direct comparison (no bit tricks), clamped to the code
    range [0, 254].  amax = 0 gives code 0.
    """
    a = np.asarray(amax, dtype=np.float64)
    if np.any(a < 0) or np.any(~np.isfinite(a)):
        raise ValueError("amax must be finite and non-negative")
    _, e = np.frexp(np.where(a > 0, a, 1.0))
    s = (e - 1) - 8                          # guess: floor(log2 a) - 8
    # adjust so that s is the smallest integer with a <= 448 * 2**s
    for _ in range(3):
        s = np.where(a > E4M3_MAX * np.ldexp(1.0, s), s + 1, s)
    for _ in range(3):
        s = np.where(a <= E4M3_MAX * np.ldexp(1.0, s - 1), s - 1, s)
    code = np.clip(s + 127, 0, 254)
    return np.where(a > 0, code, 0).astype(np.uint8)
