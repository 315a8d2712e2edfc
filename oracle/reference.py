"""Plain definitions the ring cache is pinned against (oracle; test infrastructure only).

``LinearCache`` is the launch software's semantics as the Runway Characters
post describes them in "Where the Time Went": every call keeps a time-ordered
window of the last C tokens (advanced by copying), re-applies RoPE to every
cached key and re-quantises the whole window, then attends. Its positions are
window indices, which follow time order because the window is kept in order.
Attention depends only on query-key position differences, so in exact
arithmetic it must equal the ring with write-time RoPE ("Do It Once, at Write
Time").

``SlotOrderRing`` is the combination the same section says a test pins as
invalid: ring storage with positions taken from slot indices. Before the ring
wraps slot order is time order and it agrees with ``LinearCache``; after the
wrap it does not.

``direct_attention`` is softmax attention written out with scalar loops, for
brute-force checks on tiny inputs.
"""
from __future__ import annotations

import math

import numpy as np

from . import e4m3, rope
from .cache import softmax_attention


def direct_attention(q, k, v):
    """Scalar-loop softmax attention. ``q[n,H,d]``, ``k,v[H,m,d]`` -> ``[n,H,d]``."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n, H, d = q.shape
    m = k.shape[1]
    out = np.zeros((n, H, d))
    for h in range(H):
        for i in range(n):
            s = [sum(q[i, h, t] * k[h, j, t] for t in range(d)) / math.sqrt(d) for j in range(m)]
            top = max(s)
            w = [math.exp(x - top) for x in s]
            z = sum(w)
            for t in range(d):
                out[i, h, t] = sum(w[j] * v[h, j, t] for j in range(m)) / z
    return out


class LinearCache:
    """Launch-software cache: copy-shifted window, RoPE and FP8 redone every call.

    ``mode='fp64'``: exact rotation, no quantisation.
    ``mode='fp8'``: keys rotated in fp32 at window positions, then the whole
    window quantised with the given per-head scales, on every call.
    """

    def __init__(self, heads, head_dim, capacity, rope_base=10000.0, mode="fp64",
                 scales=None):
        self.H, self.d, self.C = heads, head_dim, capacity
        self.base = rope_base
        self.mode = mode
        self.k = np.zeros((0, heads, head_dim), dtype=np.float32)
        self.v = np.zeros((0, heads, head_dim), dtype=np.float32)
        self.last_n = 0
        self.scales = scales   # [4, H] fp32 when mode == 'fp8'

    def write(self, k, v):
        k = np.asarray(k, dtype=np.float32)
        v = np.asarray(v, dtype=np.float32)
        # shift the window by copying: append the new frame, drop the oldest
        self.k = np.concatenate([self.k, k])[-self.C:].copy()
        self.v = np.concatenate([self.v, v])[-self.C:].copy()
        self.last_n = k.shape[0]

    def quantized_window(self):
        """FP8 codes of the whole window as the call re-creates them (mode 'fp8'):
        keys rotated in fp32 at window positions 0 .. m-1, then both tensors
        quantised with the per-head scales. Returns ``(k8, v8)``, each ``[m,H,d]``."""
        m = self.k.shape[0]
        sk, ik, sv, iv = self.scales
        c, s = rope.cos_sin(np.arange(m), self.d, self.base)
        kr = rope.rotate(self.k, c[:, None, :], s[:, None, :])
        return e4m3.quantize(kr, ik[None, :, None]), e4m3.quantize(self.v, iv[None, :, None])

    def attend(self, q, rows=None):
        q = np.asarray(q, dtype=np.float32)
        m = self.k.shape[0]
        kpos = np.arange(m)                        # window index = time order
        qpos = np.arange(m - self.last_n, m)
        if self.mode == "fp64":
            kr = rope.rotate64(self.k.astype(np.float64), kpos, self.d, self.base)
            qr = rope.rotate64(q.astype(np.float64), qpos, self.d, self.base)
            kk = np.transpose(kr, (1, 0, 2))
            vv = np.transpose(self.v.astype(np.float64), (1, 0, 2))
        else:
            sk, ik, sv, iv = self.scales
            k8, v8 = self.quantized_window()
            kk = np.transpose(e4m3.decode(k8) * sk.astype(np.float64)[None, :, None], (1, 0, 2))
            vv = np.transpose(e4m3.decode(v8) * sv.astype(np.float64)[None, :, None], (1, 0, 2))
            c, s = rope.cos_sin(qpos, self.d, self.base)
            qr = rope.rotate(q, c[:, None, :], s[:, None, :]).astype(np.float64)
        if rows is not None:
            qr = qr[np.asarray(rows)]
        return softmax_attention(qr, kk, vv)


class SlotOrderRing:
    """Ring storage with slot-index positions (exact arithmetic). Invalid by design."""

    def __init__(self, heads, head_dim, capacity, rope_base=10000.0):
        self.H, self.d, self.C = heads, head_dim, capacity
        self.base = rope_base
        self.k = np.zeros((capacity, heads, head_dim))
        self.v = np.zeros((capacity, heads, head_dim))
        self.tokens = 0
        self.last_slots = None

    def write(self, k, v):
        n = k.shape[0]
        slots = (self.tokens + np.arange(n)) % self.C
        self.k[slots] = rope.rotate64(np.asarray(k, np.float64), slots, self.d, self.base)
        self.v[slots] = np.asarray(v, np.float64)
        self.tokens += n
        self.last_slots = slots

    def attend(self, q):
        nv = min(self.tokens, self.C)
        qr = rope.rotate64(np.asarray(q, np.float64), self.last_slots, self.d, self.base)
        kk = np.transpose(self.k[:nv], (1, 0, 2))
        vv = np.transpose(self.v[:nv], (1, 0, 2))
        return softmax_attention(qr, kk, vv)
