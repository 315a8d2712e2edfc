"""The per-step sweep: many independent ring caches, each written and attended
once per diffusion step, in order, on one stream.

Shape of one step, as the Runway Characters post gives it ("Where the Time
Went"): the model has 60 blocks and runs 4 denoising passes per step, so a
step makes 240 attention calls; every call has a private ring (5,788 slots),
into which each step adds one frame of 757 tokens. The calls go out one by
one on a single stream, since each block consumes the previous block's
output.

Inputs are drawn on the device from per-cache seeded generators (seed
``spec.seed * 1000 + cache index``) with the production-call distribution.
``storage`` picks the cache storage for every cache (E4M3 codes, the
default, or bf16). Every cache is calibrated on its first frame and prefilled with
``spec.prefill_frames`` frames, so the ring has wrapped before the first timed
step. A timed step writes each cache's step frame at the next positions and
attends its queries over the whole ring, by default through the fused
write + attend call.
"""
from __future__ import annotations

from typing import Dict, Iterable, List

import torch

from . import workloads as W


class Sweep:
    def __init__(self, sfkv, n_caches: int = W.CALLS_PER_STEP, spec: W.WorkloadSpec = W.SWEEP,
                 keep_frames_of: Iterable[int] = (), device: str = "cuda", storage: int = 0):
        s = spec.shape
        self.spec = spec
        self.sfkv = sfkv
        self.n = s.new_tokens
        self.rope = sfkv.Rope(s.head_dim, s.max_position, s.rope_base, device=device)
        self.caches = [sfkv.RingCache(self.rope, s.heads, s.capacity, s.new_tokens, device=device,
                                      storage=storage)
                       for _ in range(n_caches)]
        need = self.caches[0].workspace_bytes()
        # one workspace serves every call: the calls are ordered on one stream
        self.workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=device)
        self.outs = [torch.empty(self.n, s.heads, s.head_dim, dtype=torch.float32, device=device)
                     for _ in range(n_caches)]
        self.gens = [W.FrameStream(spec, seed=spec.seed * 1000 + i, device=device)
                     for i in range(n_caches)]
        self.keep = set(keep_frames_of)
        self.kept: Dict[int, List] = {i: [] for i in self.keep}
        self.frames = [None] * n_caches

    def _draw(self, i):
        q, k, v = self.gens[i].frame(self.n)
        if i in self.keep:
            self.kept[i].append((q.cpu(), k.cpu(), v.cpu()))
        return q, k, v

    def prefill(self):
        """Calibrate each cache on its first frame, write the prefill frames, then
        draw (and keep resident) the frame every timed step writes."""
        for i, c in enumerate(self.caches):
            for f in range(self.spec.prefill_frames):
                q, k, v = self._draw(i)
                if f == 0:
                    c.calibrate_scales(k, v)
                c.cache_write(k, v)
            self.frames[i] = self._draw(i)

    def positions_left(self) -> int:
        st = self.caches[0].state()
        return (self.rope.max_position - st["next_pos"]) // self.n

    def step(self, stream=None, fused: bool = True):
        """One diffusion step: write + attend on every cache, in order, as one
        fused call per cache (or, with fused=False, cache_write then attend)."""
        for c, (q, k, v), out in zip(self.caches, self.frames, self.outs):
            if fused:
                self.sfkv.write_attend(c.handle, k, v, q, out, self.workspace, stream)
            else:
                c.cache_write(k, v, stream)
                self.sfkv.attend(c.handle, q, out, self.workspace, stream)

    def reset_all(self, stream=None):
        """Position reset of every cache (each back to position 0): one delta
        rotation per cache, all issued through one batched call."""
        self.sfkv.rebase_positions_many([c.handle for c in self.caches],
                                        [c.state()["next_pos"] for c in self.caches], stream)
