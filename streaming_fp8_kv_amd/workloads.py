"""Seeded synthetic workloads for the streaming FP8 ring KV cache.

This module only draws random numbers and names shapes. It holds none of the
method's arithmetic (no RoPE, no quantisation, no attention), so both the HIP
path and the CPU oracle can be fed from it without sharing any computation.

The shapes follow the production call described in the Runway Characters post
("Where the Time Went"): every attention call owns a cache of 5,788 slots of
which 757 are new per step, and one step is 60 blocks x 4 denoising passes =
240 calls. Head count, head dimension and value distributions are not on the
pages; they are fixed here as synthetic stand-ins for the model's activations.

Draw order for one cache stream (all from one ``torch.Generator`` seeded with
the stream's seed):

1. per-head standard deviations for Q, then K, then V (``heads`` values each,
   uniform on the configured range; skipped when the range is ``None``);
2. then, frame by frame, Q, K, V of shape ``[n, heads, head_dim]``.

Normal draws use ``torch.randn``. Student-t(3) draws are built from four
independent normals as ``z0 / sqrt((z1^2 + z2^2 + z3^2) / 3)``, which is the
textbook construction of a t variable with three degrees of freedom.
"""
from __future__ import annotations

import dataclasses
from typing import Optional, Tuple

import torch

__all__ = [
    "CacheShape", "WorkloadSpec", "FrameStream",
    "TINY", "PROD", "SWEEP", "LONG", "STRESS", "ALL_SPECS",
    "BLOCKS", "PASSES", "CALLS_PER_STEP", "RESET_PERIOD",
]

# Structure of one diffusion step and the reset schedule, from the Runway
# Characters post ("Where the Time Went"; "Do It Once, at Write Time").
BLOCKS = 60
PASSES = 4
CALLS_PER_STEP = BLOCKS * PASSES  # 240
RESET_PERIOD = 42


@dataclasses.dataclass(frozen=True)
class CacheShape:
    heads: int
    head_dim: int
    capacity: int          # ring slots
    new_tokens: int        # tokens per steady-state write
    rope_base: float = 10000.0
    max_position: int = 65536


@dataclasses.dataclass(frozen=True)
class WorkloadSpec:
    name: str
    shape: CacheShape
    seed: int
    dtype: torch.dtype                      # input dtype of Q/K/V
    dist: str                               # "normal" or "t3"
    sigma_q: Optional[Tuple[float, float]]  # per-head std range for Q
    sigma_kv: Optional[Tuple[float, float]]  # per-head std range for K and V
    steps: int                              # writes in the session
    prefill_frames: int = 0                 # frames written before the timed one
    reset_period: int = 0                   # 0 = never rebase
    calls: int = 1                          # independent caches (the sweep)
    first_tokens: Optional[Tuple[int, int]] = None  # range of the first write's length


TINY = WorkloadSpec(
    name="tiny_h1_d64_n16_c64", shape=CacheShape(1, 64, 64, 16, max_position=1024),
    seed=1, dtype=torch.float32, dist="normal", sigma_q=None, sigma_kv=None,
    steps=10, reset_period=3)
PROD = WorkloadSpec(
    name="call_h24_d128_n757_c5788", shape=CacheShape(24, 128, 5788, 757),
    seed=2, dtype=torch.bfloat16, dist="normal", sigma_q=(0.5, 4.0),
    sigma_kv=(0.5, 4.0), steps=9, prefill_frames=8)
SWEEP = dataclasses.replace(
    PROD, name="step_240x_h24_d128_n757_c5788", seed=3, calls=CALLS_PER_STEP)
LONG = dataclasses.replace(
    PROD, name="session200_h24_d128_n757_c5788_reset42", seed=4, steps=200,
    prefill_frames=0, reset_period=RESET_PERIOD,
    shape=dataclasses.replace(PROD.shape, max_position=32768))
STRESS = WorkloadSpec(
    name="stress_h40_d128_t3_c5788", shape=CacheShape(40, 128, 5788, 757),
    seed=5, dtype=torch.bfloat16, dist="t3", sigma_q=(0.5, 4.0),
    sigma_kv=(0.5, 8.0), steps=51, first_tokens=(100, 757))

ALL_SPECS = (TINY, PROD, SWEEP, LONG, STRESS)


class FrameStream:
    """Frames of one cache, drawn in a fixed order from one seeded generator.

    ``device`` selects where the generator lives. CPU streams are what the
    parity tests use (the oracle sees the identical host tensors); a CUDA
    stream draws the same distribution on the device for the benchmark, where
    hundreds of caches would be too slow to draw on the host.
    """

    def __init__(self, spec: WorkloadSpec, seed: Optional[int] = None,
                 device: str = "cpu"):
        self.spec = spec
        self.device = torch.device(device)
        self.gen = torch.Generator(device=self.device)
        self.gen.manual_seed(spec.seed if seed is None else seed)
        h = spec.shape.heads
        self.sigma_q = self._sigmas(spec.sigma_q, h)
        self.sigma_k = self._sigmas(spec.sigma_kv, h)
        self.sigma_v = self._sigmas(spec.sigma_kv, h)
        self.frames_drawn = 0

    def _sigmas(self, rng, h):
        if rng is None:
            return None
        lo, hi = rng
        return torch.empty(h, device=self.device).uniform_(lo, hi, generator=self.gen)

    def first_length(self) -> int:
        """Length of the session's first write (drawn only when configured)."""
        s = self.spec
        if s.first_tokens is None:
            return s.shape.new_tokens
        lo, hi = s.first_tokens
        return int(torch.randint(lo, hi + 1, (1,), generator=self.gen,
                                 device=self.device).item())

    def _normal(self, n):
        s = self.spec.shape
        return torch.randn(n, s.heads, s.head_dim, generator=self.gen,
                           device=self.device, dtype=torch.float32)

    def _t3(self, n):
        z = [self._normal(n) for _ in range(4)]
        chi2 = z[1] * z[1] + z[2] * z[2] + z[3] * z[3]
        return z[0] / torch.sqrt(chi2 / 3.0)

    def _draw(self, n, sigma, heavy):
        x = self._t3(n) if heavy else self._normal(n)
        if sigma is not None:
            x = x * sigma[None, :, None]
        return x.to(self.spec.dtype)

    def frame(self, n: Optional[int] = None):
        """Return ``(q, k, v)``, each ``[n, heads, head_dim]`` in the spec dtype."""
        if n is None:
            n = self.spec.shape.new_tokens
        heavy = self.spec.dist == "t3"
        q = self._draw(n, self.sigma_q, False)
        k = self._draw(n, self.sigma_k, heavy)
        v = self._draw(n, self.sigma_v, heavy)
        self.frames_drawn += 1
        return q, k, v
