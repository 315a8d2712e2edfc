"""OCP E4M3FN codec (oracle; test infrastructure only).

The pages say the cache is quantised to FP8 with per-head scales (Runway
Characters post, "Do It Once, at Write Time"; "Blackwell and Beyond Four
GPUs") but name neither the FP8 variant nor its rounding. Reading taken: OCP
E4M3FN (1 sign, 4 exponent bits with bias 7, 3 mantissa bits; no infinities;
0x7F/0xFF are NaN; largest finite 448), with values clamped to [-448, 448]
first and then rounded to nearest, ties to even.

Pinned by: the closed-form decode of all 256 codes, exhaustive round trips,
every midpoint between adjacent codes (and one fp32 ulp either side), a
brute-force nearest-code search, and torch's float8_e4m3fn conversion.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


def decode_table() -> np.ndarray:
    """All 256 codes as fp64 (NaN for 0x7F and 0xFF); the closed form."""
    out = np.empty(256, dtype=np.float64)
    for code in range(256):
        sign = -1.0 if code & 0x80 else 1.0
        e = (code >> 3) & 0xF
        m = code & 0x7
        if e == 0xF and m == 0x7:
            out[code] = np.nan
        elif e == 0:
            out[code] = sign * m * 2.0 ** -9          # subnormal: m/8 * 2^(1-7)
        else:
            out[code] = sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return out


_DECODE = decode_table()


def decode(codes: np.ndarray) -> np.ndarray:
    """uint8 codes -> fp64 values (exact)."""
    return _DECODE[np.asarray(codes, dtype=np.uint8)]


def encode(x: np.ndarray) -> np.ndarray:
    """fp32 values -> uint8 codes: clamp to +-448, then round to nearest even.

    Works in fp64, where every step below is exact for fp32 inputs:
      * |y| < 2^-6 is the subnormal range: the code is rint(|y| * 2^9), which
        may reach 8, the bit pattern of the smallest normal 2^-6;
      * otherwise |y| = t * 2^E with t in [1, 2); the mantissa field is
        rint((t - 1) * 8), and a result of 8 carries into the exponent field
        just as the bit pattern requires.
    The sign bit is taken from the clamped value, so -0.0 encodes as 0x80.
    """
    y = np.clip(np.asarray(x, dtype=np.float32).astype(np.float64), -E4M3_MAX, E4M3_MAX)
    a = np.abs(y)
    sign = np.signbit(y).astype(np.int64) << 7
    sub = a < 2.0 ** -6
    code = np.empty(a.shape, dtype=np.int64)
    code[sub] = np.rint(a[sub] * 512.0).astype(np.int64)
    f, e2 = np.frexp(a[~sub])                  # a = f * 2^e2, f in [0.5, 1)
    ex = e2 - 1                                # a = t * 2^ex, t in [1, 2)
    t = f * 2.0
    mant = np.rint((t - 1.0) * 8.0).astype(np.int64)
    code[~sub] = ((ex + 7) << 3) + mant
    return (code | sign).astype(np.uint8)


def quantize(x: np.ndarray, inv_scale) -> np.ndarray:
    """Multiply by the inverse scale in fp32 (one rounding), then encode.

    ``inv_scale`` broadcasts against ``x``; this is the write-time quantiser.
    """
    y = np.asarray(x, dtype=np.float32) * np.asarray(inv_scale, dtype=np.float32)
    return encode(y.astype(np.float32))
