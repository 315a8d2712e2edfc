"""bfloat16 codec (oracle; test infrastructure only).

The pages contrast the FP8 cache with a non-FP8 one ("Blackwell and Beyond Four
GPUs": the FP8 cache saves time on H100 and costs time on B200). Reading taken
for the non-FP8 variant: the ring stores bfloat16 (1 sign, 8 exponent and 7
mantissa bits, the top half of an IEEE fp32), rounded from fp32 to nearest,
ties to even, with no saturation (bf16 shares fp32's range).

Pinned by: the closed-form decode (a bf16 is the fp32 whose low 16 bits are
zero), torch's bfloat16 conversion on random, tie, subnormal and extreme
values, and exact round trips of every bf16 value with a finite exponent.
"""
from __future__ import annotations

import numpy as np


def decode(bits: np.ndarray) -> np.ndarray:
    """uint16 bf16 bit patterns -> float32 (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)


def encode(x: np.ndarray) -> np.ndarray:
    """float32 -> uint16 bf16, round to nearest, ties to even (finite inputs)."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return r.astype(np.uint16)
