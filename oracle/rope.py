"""Rotary position embedding (oracle; test infrastructure only).

The pages apply RoPE to keys once, at write time, and rotate the cached window
by a single delta at each position reset (Runway Characters post, "Do It Once,
at Write Time"), but give neither the RoPE variant nor its base. Reading taken:
1-D RoPE over the whole head dimension with interleaved pairs
(x[2i], x[2i+1]), frequency theta_i = base^(-2i/d), base 10000.

Table: angle = p * theta_i in fp64; cos and sin from the C library in fp64
(``math.cos``/``math.sin``, which call libm), each rounded once to fp32.
Rotation in fp32 with every product and sum rounded separately (no fused
multiply-add), so a bit-exact comparison with another IEEE implementation of
the same formula is possible:
    a' = fl(fl(a*c) - fl(b*s)),   b' = fl(fl(a*s) + fl(b*c)).

Pinned by: R(0) = identity, per-pair norm preservation, agreement with complex
multiplication x * exp(i p theta) in complex128, the composition law
R(a)^T R(b) = R(b - a) in fp64, and a table check against numpy's own cos/sin.
"""
from __future__ import annotations

import math

import numpy as np


def inv_freq(head_dim: int, base: float = 10000.0) -> np.ndarray:
    """theta_i = base ** ((-2.0 * i) / head_dim), i = 0 .. head_dim/2 - 1 (fp64)."""
    return np.array([base ** ((-2.0 * i) / head_dim) for i in range(head_dim // 2)],
                    dtype=np.float64)


_ROWS: dict = {}


def _row(pos: int, head_dim: int, base: float):
    memo = _ROWS.setdefault((head_dim, base), {})
    r = memo.get(pos)
    if r is None:
        th = inv_freq(head_dim, base)
        c = np.empty(head_dim // 2, dtype=np.float32)
        s = np.empty(head_dim // 2, dtype=np.float32)
        for i in range(head_dim // 2):
            ang = float(pos) * float(th[i])
            c[i] = np.float32(math.cos(ang))
            s[i] = np.float32(math.sin(ang))
        r = (c, s)
        memo[pos] = r
    return r


def cos_sin(positions, head_dim: int, base: float = 10000.0):
    """fp32 (cos, sin), each ``[len(positions), head_dim/2]``, one row per position.

    Rows are computed on first use and memoised, so only the positions a test
    touches are ever evaluated.
    """
    pos = np.atleast_1d(np.asarray(positions, dtype=np.int64))
    c = np.empty((pos.size, head_dim // 2), dtype=np.float32)
    s = np.empty((pos.size, head_dim // 2), dtype=np.float32)
    for j, p in enumerate(pos.tolist()):
        c[j], s[j] = _row(int(p), int(head_dim), float(base))
    return c, s


def rotate(x: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    """Rotate interleaved pairs of ``x[..., d]`` (fp32) by per-pair (cos, sin).

    ``cos``/``sin`` broadcast against ``x[..., d/2]``. Every operation is a
    separately rounded numpy fp32 ufunc, so no fused multiply-add occurs.
    """
    x = np.asarray(x, dtype=np.float32)
    a = x[..., 0::2]
    b = x[..., 1::2]
    c = np.asarray(cos, dtype=np.float32)
    s = np.asarray(sin, dtype=np.float32)
    ac = a * c
    bs = b * s
    as_ = a * s
    bc = b * c
    out = np.empty_like(x)
    out[..., 0::2] = ac - bs
    out[..., 1::2] = as_ + bc
    return out


def rotate_back(x: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    """Rotate pairs by the negative angle: a' = fl(fl(a*c) + fl(b*s)),
    b' = fl(fl(b*c) - fl(a*s)). This is the delta rotation of a rebase."""
    x = np.asarray(x, dtype=np.float32)
    a = x[..., 0::2]
    b = x[..., 1::2]
    c = np.asarray(cos, dtype=np.float32)
    s = np.asarray(sin, dtype=np.float32)
    out = np.empty_like(x)
    out[..., 0::2] = a * c + b * s
    out[..., 1::2] = b * c - a * s
    return out


def rotate64(x: np.ndarray, pos: np.ndarray, head_dim: int, base: float = 10000.0) -> np.ndarray:
    """Exact-arithmetic rotation in fp64 (for the fp64 reference modes).

    ``x[..., n, H, d]`` with ``pos[n]`` (may be negative); angle = pos*theta_i.
    """
    x = np.asarray(x, dtype=np.float64)
    th = inv_freq(head_dim, base)
    ang = np.asarray(pos, dtype=np.float64)[:, None] * th[None, :]   # [n, d/2]
    c = np.cos(ang)[:, None, :]
    s = np.sin(ang)[:, None, :]
    a = x[..., 0::2]
    b = x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = a * c - b * s
    out[..., 1::2] = a * s + b * c
    return out
