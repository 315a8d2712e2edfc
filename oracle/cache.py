"""The ring KV cache, computed plainly on the CPU (oracle; test infrastructure only).

Source: Runway Characters post, "Do It Once, at Write Time": RoPE and FP8
quantisation are applied to each new frame once, as it enters the cache, with
per-head scales calibrated once per session; the cache is a ring, so the
window advances without copying; at each position reset one delta rotation is
applied to the cached window; once the ring wraps, positions must follow time,
not slot order. "Where the Time Went" fixes the shape of one call (5,788
slots, 757 new) and that every call reads its own cache.

Readings where the pages are silent (each listed in the design notes):
  * the ring is token-granular: global token t lives in slot t mod C, and
    after T tokens the ring holds tokens [T - min(T, C), T);
  * position of token t is t - B, with B the sum of all rebase deltas so far;
  * scales are calibrated from the first write's data, on post-RoPE keys and
    raw values: scale = absmax / 448 and inv = 448 / absmax, both divided in
    fp64 and rounded once to fp32 (1 and 1 when absmax is 0);
  * attention has no mask and uses 1/sqrt(d); the queries are the last
    write's tokens, rotated at that write's positions;
  * a rebase rotates the stored FP8 codes by -delta in the code domain (the
    per-head scale cancels, since rotation is linear), clamps and re-encodes.

Three modes:
  ``fp8``  the bit-exact pipeline: fp32 rotation without fused multiply-add,
           one fp32 multiply by the inverse scale, clamp, round-to-nearest-even
           E4M3; attention then in fp64 on the decoded cache.
  ``bf16`` the non-FP8 variant ("Blackwell and Beyond Four GPUs" weighs the
           FP8 cache against one without FP8): the same fp32 rotation, then
           keys and values rounded to bfloat16 (nearest, ties to even); no
           quantisation scale enters the values, so calibration only marks the
           session as started; attention is in fp64 on the bf16 values.
  ``fp64`` the same ring with exact arithmetic and no quantisation, used to pin
           the ring against the plain linear definition.

Parity: pinned (see the oracle tests) by closed forms for slots and positions,
by the linear read-time-RoPE cache, by re-rotation from scratch, and by direct
softmax attention on small inputs.
"""
from __future__ import annotations

import math
from typing import Optional

import numpy as np

from . import bf16, e4m3, rope


class RingCache:
    def __init__(self, heads: int, head_dim: int, capacity: int,
                 max_new_tokens: Optional[int] = None, rope_base: float = 10000.0,
                 max_position: int = 65536, mode: str = "fp8"):
        if mode not in ("fp8", "bf16", "fp64"):
            raise ValueError("mode must be 'fp8', 'bf16' or 'fp64'")
        if head_dim % 2:
            raise ValueError("head_dim must be even")
        self.H, self.d, self.C = int(heads), int(head_dim), int(capacity)
        self.max_new = int(max_new_tokens) if max_new_tokens else self.C
        if not 1 <= self.max_new <= self.C:
            raise ValueError("max_new_tokens must be in [1, capacity]")
        self.base = float(rope_base)
        self.max_position = int(max_position)
        self.mode = mode
        if mode == "fp8":
            self.k = np.zeros((self.H, self.C, self.d), dtype=np.uint8)
            self.v = np.zeros((self.H, self.C, self.d), dtype=np.uint8)
        elif mode == "bf16":
            self.k = np.zeros((self.H, self.C, self.d), dtype=np.uint16)
            self.v = np.zeros((self.H, self.C, self.d), dtype=np.uint16)
        else:
            self.k = np.zeros((self.H, self.C, self.d), dtype=np.float64)
            self.v = np.zeros((self.H, self.C, self.d), dtype=np.float64)
        self.pos = np.zeros(self.C, dtype=np.int64)
        self.tokens = 0          # T: tokens written in the session
        self.next_pos = 0        # position the next token will get
        self.last_pos0 = None    # first position of the most recent write
        self.last_n = 0
        self.scale_k = self.inv_k = self.scale_v = self.inv_v = None
        self.calibrated = False

    # ---- ring bookkeeping (integer, exact) --------------------------------
    @property
    def write_slot(self) -> int:
        return self.tokens % self.C

    @property
    def n_valid(self) -> int:
        return min(self.tokens, self.C)

    def valid_slots(self) -> np.ndarray:
        return np.arange(self.n_valid, dtype=np.int64)

    def time_order(self) -> np.ndarray:
        """Valid slots listed from the oldest token to the newest."""
        t0 = self.tokens - self.n_valid
        return (np.arange(t0, self.tokens, dtype=np.int64)) % self.C

    # ---- calibration ------------------------------------------------------
    @staticmethod
    def _scale_pair(m: float):
        if m == 0.0:
            return np.float32(1.0), np.float32(1.0)
        return np.float32(float(m) / 448.0), np.float32(448.0 / float(m))

    def calibrate(self, k, v):
        """Per-head scales from one frame ``[n, H, d]`` at the next write's positions."""
        k = np.asarray(k, dtype=np.float32)
        v = np.asarray(v, dtype=np.float32)
        n = self._check_frame(k, v)
        if self.mode == "fp64":
            raise ValueError("fp64 mode has no quantisation scales")
        self._check_positions(n)
        self.calibrated = True
        if self.mode == "bf16":
            return                      # bf16 storage carries no scale
        c, s = rope.cos_sin(self.next_pos + np.arange(n), self.d, self.base)
        kr = rope.rotate(k, c[:, None, :], s[:, None, :])
        mk = np.abs(kr).max(axis=(0, 2))
        mv = np.abs(v).max(axis=(0, 2))
        sk, ik, sv, iv = [], [], [], []
        for h in range(self.H):
            a, b = self._scale_pair(float(mk[h]))
            sk.append(a); ik.append(b)
            a, b = self._scale_pair(float(mv[h]))
            sv.append(a); iv.append(b)
        self.scale_k = np.array(sk, dtype=np.float32)
        self.inv_k = np.array(ik, dtype=np.float32)
        self.scale_v = np.array(sv, dtype=np.float32)
        self.inv_v = np.array(iv, dtype=np.float32)

    def scales(self) -> np.ndarray:
        """``[4, H]`` fp32: scale_k, inv_k, scale_v, inv_v (fp8 mode)."""
        if self.mode != "fp8":
            raise ValueError("only the fp8 mode has quantisation scales")
        return np.stack([self.scale_k, self.inv_k, self.scale_v, self.inv_v])

    # ---- write --------------------------------------------------------------
    def _check_frame(self, k, v) -> int:
        if k.ndim != 3 or k.shape[1:] != (self.H, self.d) or v.shape != k.shape:
            raise ValueError("frames must be [n, heads, head_dim]")
        n = k.shape[0]
        if not 1 <= n <= self.max_new:
            raise ValueError("n_tokens must be in [1, max_new_tokens]")
        return n

    def _check_positions(self, n):
        if self.next_pos + n > self.max_position:
            raise OverflowError("write positions would reach max_position")

    def write(self, k, v):
        """Rotate, quantise and store one frame; advance the ring."""
        k = np.asarray(k, dtype=np.float32)
        v = np.asarray(v, dtype=np.float32)
        n = self._check_frame(k, v)
        self._check_positions(n)
        pos = self.next_pos + np.arange(n, dtype=np.int64)
        slots = (self.tokens + np.arange(n, dtype=np.int64)) % self.C
        if self.mode == "fp8":
            if self.inv_k is None:
                raise RuntimeError("write before calibrate")
            c, s = rope.cos_sin(pos, self.d, self.base)
            kr = rope.rotate(k, c[:, None, :], s[:, None, :])            # [n, H, d]
            k8 = e4m3.quantize(kr, self.inv_k[None, :, None])
            v8 = e4m3.quantize(v, self.inv_v[None, :, None])
            self.k[:, slots, :] = np.transpose(k8, (1, 0, 2))
            self.v[:, slots, :] = np.transpose(v8, (1, 0, 2))
        elif self.mode == "bf16":
            if not self.calibrated:
                raise RuntimeError("write before calibrate")
            c, s = rope.cos_sin(pos, self.d, self.base)
            kr = rope.rotate(k, c[:, None, :], s[:, None, :])
            self.k[:, slots, :] = np.transpose(bf16.encode(kr), (1, 0, 2))
            self.v[:, slots, :] = np.transpose(bf16.encode(v), (1, 0, 2))
        else:
            kr = rope.rotate64(k.astype(np.float64), pos, self.d, self.base)
            self.k[:, slots, :] = np.transpose(kr, (1, 0, 2))
            self.v[:, slots, :] = np.transpose(v.astype(np.float64), (1, 0, 2))
        self.pos[slots] = pos
        self.tokens += n
        self.next_pos += n
        self.last_pos0, self.last_n = int(pos[0]), n

    # ---- attend -------------------------------------------------------------
    def dequantized(self):
        """Valid cache as fp64 ``(k, v)``, each ``[H, n_valid, d]`` (scales applied)."""
        nv = self.n_valid
        if self.mode == "fp8":
            kk = e4m3.decode(self.k[:, :nv, :]) * self.scale_k.astype(np.float64)[:, None, None]
            vv = e4m3.decode(self.v[:, :nv, :]) * self.scale_v.astype(np.float64)[:, None, None]
        elif self.mode == "bf16":
            kk = bf16.decode(self.k[:, :nv, :]).astype(np.float64)
            vv = bf16.decode(self.v[:, :nv, :]).astype(np.float64)
        else:
            kk, vv = self.k[:, :nv, :], self.v[:, :nv, :]
        return kk, vv

    def rotated_queries(self, q) -> np.ndarray:
        """The last write's queries rotated at its positions (fp32 in fp8 and bf16 modes)."""
        q = np.asarray(q, dtype=np.float32)
        if self.last_pos0 is None:
            raise RuntimeError("attend before any write")
        if q.ndim != 3 or q.shape != (self.last_n, self.H, self.d):
            raise ValueError("queries must be the last write's [n, heads, head_dim]")
        pos = self.last_pos0 + np.arange(self.last_n, dtype=np.int64)
        if self.mode in ("fp8", "bf16"):
            c, s = rope.cos_sin(pos, self.d, self.base)
            return rope.rotate(q, c[:, None, :], s[:, None, :]).astype(np.float64)
        return rope.rotate64(q.astype(np.float64), pos, self.d, self.base)

    def attend(self, q, rows=None) -> np.ndarray:
        """softmax(q k^T / sqrt(d)) v over every valid slot; fp64 ``[rows, H, d]``.

        ``rows`` selects query rows (all by default), so large calls can be
        checked on a sample.
        """
        qr = self.rotated_queries(q)
        if rows is not None:
            qr = qr[np.asarray(rows, dtype=np.int64)]
        kk, vv = self.dequantized()
        return softmax_attention(qr, kk, vv)

    # ---- rebase -------------------------------------------------------------
    def rebase(self, delta: int):
        """Shift every position down by ``delta`` with one rotation of the keys."""
        delta = int(delta)
        if delta < 0 or delta > self.next_pos:
            raise OverflowError("delta must be in [0, next_pos]")
        nv = self.n_valid
        if self.mode == "fp8":
            c, s = rope.cos_sin([delta], self.d, self.base)
            x = e4m3.decode(self.k[:, :nv, :]).astype(np.float32)          # exact
            y = rope.rotate_back(x, c[0], s[0])
            self.k[:, :nv, :] = e4m3.encode(y)
        elif self.mode == "bf16":
            c, s = rope.cos_sin([delta], self.d, self.base)
            x = bf16.decode(self.k[:, :nv, :])                                 # exact
            self.k[:, :nv, :] = bf16.encode(rope.rotate_back(x, c[0], s[0]))
        else:
            pos = np.full(nv, -delta, dtype=np.int64)
            kt = np.transpose(self.k[:, :nv, :], (1, 0, 2))                 # [nv, H, d]
            self.k[:, :nv, :] = np.transpose(rope.rotate64(kt, pos, self.d, self.base), (1, 0, 2))
        self.pos[:nv] -= delta
        self.next_pos -= delta
        if self.last_pos0 is not None:
            self.last_pos0 -= delta


def softmax_attention(q, k, v) -> np.ndarray:
    """Plain softmax attention per head in fp64.

    ``q[n, H, d]``, ``k[H, m, d]``, ``v[H, m, d]`` -> ``[n, H, d]``. Scores are
    q.k / sqrt(d); the row maximum is subtracted before exp (which leaves the
    softmax unchanged) and the weighted sum is divided by the sum of weights.
    """
    q = np.asarray(q, dtype=np.float64)
    n, H, d = q.shape
    out = np.empty((n, H, d), dtype=np.float64)
    inv_sqrt_d = 1.0 / math.sqrt(d)
    for h in range(H):
        s = (q[:, h, :] @ k[h].T) * inv_sqrt_d                             # [n, m]
        s -= s.max(axis=1, keepdims=True)
        p = np.exp(s)
        out[:, h, :] = (p @ v[h]) / p.sum(axis=1, keepdims=True)
    return out
