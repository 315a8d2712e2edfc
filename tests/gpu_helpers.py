"""Shared pieces of the GPU parity tests: a GPU cache driven in lockstep with its
oracle twin, and the attention error metric.

Parity bar (fixed here, used by every GPU test):
  * stored code bytes (FP8, or bf16 in the non-FP8 storage), ring positions,
    scales and ring counters: bit-exact;
  * attention, per call over the checked rows: max|o - r| / max|r| <= 2e-2 and
    mean|o - r| / mean|r| <= 1e-3, where r is the oracle's fp64 attention fed the
    GPU's own cache (codes and scales).
"""
from __future__ import annotations

import sys

import numpy as np
import torch

from oracle import bf16, e4m3, rope as orope
from oracle.cache import RingCache as OracleCache, softmax_attention

A_MAX = 2e-2
B_MEAN = 1e-3


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def attention_error(out: np.ndarray, ref: np.ndarray):
    err = np.abs(out.astype(np.float64) - ref)
    return float(err.max() / np.abs(ref).max()), float(err.mean() / np.abs(ref).mean())


class Mirror:
    """One GPU ring cache and an oracle cache over a subset of its heads."""

    def __init__(self, sfkv, rope, spec, heads=None, max_new=None, storage="fp8"):
        s = spec.shape
        self.spec = spec
        self.H, self.d, self.C = s.heads, s.head_dim, s.capacity
        self.heads = list(range(s.heads)) if heads is None else list(heads)
        self.bf16 = storage == "bf16"
        max_new = max_new or s.new_tokens
        self.gpu = sfkv.RingCache(rope, s.heads, s.capacity, max_new,
                                  storage=sfkv.STORE_BF16 if self.bf16 else sfkv.STORE_E4M3)
        self.ora = OracleCache(len(self.heads), s.head_dim, s.capacity, max_new, s.rope_base,
                               rope.max_position, mode=storage)

    def codes(self, which, nv=None):
        """GPU codes of the checked heads as numpy (uint16 bf16 bit patterns or uint8)."""
        hs = torch.tensor(self.heads)
        t = (self.gpu.k_codes() if which == "k" else self.gpu.v_codes())[hs]
        if nv is not None:
            t = t[:, :nv]
        a = t.cpu().numpy()
        return a.view(np.uint16) if self.bf16 else a

    def _sub(self, t):
        return t[:, self.heads, :].float().numpy()

    def calibrate(self, k, v):
        self.gpu.calibrate_scales(k.cuda(), v.cuda())
        if self.bf16:
            self.factors = bf16_staging_factors(self._sub(k), self._sub(v), self.ora.next_pos,
                                                self.spec.shape.rope_base)
        self.ora.calibrate(self._sub(k), self._sub(v))

    def write(self, k, v):
        self.gpu.cache_write(k.cuda(), v.cuda())
        self.ora.write(self._sub(k), self._sub(v))

    def rebase(self, delta):
        self.gpu.rebase_positions(delta)
        self.ora.rebase(delta)

    def check_cache(self, tag=""):
        torch.cuda.synchronize()
        st = self.gpu.state()
        assert st == {"tokens": self.ora.tokens, "next_pos": self.ora.next_pos,
                      "write_slot": self.ora.write_slot, "n_valid": self.ora.n_valid}, tag
        hs = torch.tensor(self.heads)
        k8 = self.codes("k")
        v8 = self.codes("v")
        nv = self.ora.n_valid
        bad_k = np.count_nonzero(k8[:, :nv] != self.ora.k[:, :nv])
        bad_v = np.count_nonzero(v8[:, :nv] != self.ora.v[:, :nv])
        assert bad_k == 0 and bad_v == 0, f"{tag}: {bad_k} K and {bad_v} V code bytes differ"
        pos = self.gpu.positions().cpu().numpy()
        assert np.array_equal(pos[:nv], self.ora.pos[:nv]), f"{tag}: positions differ"
        sc = self.gpu.scales()[:, hs].cpu().numpy()
        want = self.factors if self.bf16 else self.ora.scales()
        assert np.array_equal(sc, want), f"{tag}: scales differ"

    def reference_from_gpu_cache(self, q, rows):
        """Oracle attention over the GPU's own codes and scales (checked heads)."""
        hs = torch.tensor(self.heads)
        nv = self.ora.n_valid
        k8 = self.codes("k", nv)
        v8 = self.codes("v", nv)
        if self.bf16:
            # bf16 storage carries no quantisation scale
            kk = bf16.decode(k8).astype(np.float64)
            vv = bf16.decode(v8).astype(np.float64)
        else:
            sc = self.gpu.scales()[:, hs].cpu().numpy().astype(np.float64)
            kk = e4m3.decode(k8) * sc[0][:, None, None]
            vv = e4m3.decode(v8) * sc[2][:, None, None]
        qr = self.ora.rotated_queries(self._sub(q))[rows]
        return softmax_attention(qr, kk, vv)

    def check_attend(self, q, rows=None, tag=""):
        out = self.gpu.attend(q.cuda())
        torch.cuda.synchronize()
        n = q.shape[0]
        rows = np.arange(n) if rows is None else np.asarray(rows)
        got = out[torch.as_tensor(rows)][:, self.heads].cpu().numpy()
        ref = self.reference_from_gpu_cache(q, rows)
        a, b = attention_error(got, ref)
        full = out.cpu().numpy()
        assert np.isfinite(full).all(), f"{tag}: non-finite attention output"
        say(f"  {tag}: attention A={a:.2e} B={b:.2e} over {len(rows)} rows x {len(self.heads)} heads")
        assert a <= A_MAX and b <= B_MEAN, f"{tag}: A={a:.3e} (bar {A_MAX}) B={b:.3e} (bar {B_MEAN})"
        return out


def bf16_staging_factors(k, v, pos0, base):
    """Expected scale slots of a bf16-storage cache after calibration on frame
    (k, v) ``[n, H, d]`` at positions pos0..: per head and tensor the power of two
    2^e with the frame's absmax in [1, 2) * 2^e (keys rotated as written), as
    ``[4, H]`` (2^e_k, 2^-e_k, 2^e_v, 2^-e_v); 1 and 1 for an all-zero head.

    These are the library's own contract for the non-FP8 storage (the factor by
    which its attention moves bf16 values into fp16 range), not part of the
    method, so they are written out here rather than in the oracle."""
    k = np.asarray(k, np.float32)
    v = np.asarray(v, np.float32)
    n, H, d = k.shape
    c, s_ = orope.cos_sin(pos0 + np.arange(n), d, base)
    kr = orope.rotate(k, c[:, None, :], s_[:, None, :])
    out = np.ones((4, H), np.float32)
    for row, x in ((0, kr), (2, v)):
        m = np.abs(x).max(axis=(0, 2)).astype(np.float64)
        for h in range(H):
            if m[h] > 0:
                e = int(np.floor(np.log2(m[h])))
                if 2.0 ** e > m[h]:
                    e -= 1
                elif 2.0 ** (e + 1) <= m[h]:
                    e += 1
                e = min(max(e, -126), 127)
                out[row, h] = np.float32(2.0 ** e)
                out[row + 1, h] = np.float32(2.0 ** -e)
    return out


def spread_rows(n, k):
    """k query rows spread over [0, n), always including the first and last."""
    if k >= n:
        return np.arange(n)
    r = np.unique(np.linspace(0, n - 1, k).round().astype(np.int64))
    return r
