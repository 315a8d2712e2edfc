"""Pins of the oracle ring cache: slot and position closed forms, the ring against the
launch software's linear cache, delta rotation against re-rotation from scratch, and the
slot-order-positions combination as invalid."""
import json
import os

import numpy as np
import pytest

from oracle import e4m3, rope
from oracle.cache import RingCache, softmax_attention
from oracle.reference import LinearCache, SlotOrderRing
from streaming_fp8_kv_amd import workloads as W

pytestmark = pytest.mark.cpu
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rel(a, b):
    return float(np.max(np.abs(a - b)) / np.max(np.abs(b)))


def tiny_frames(steps=10, seed=None):
    fs = W.FrameStream(W.TINY, seed=seed)
    return [tuple(t.numpy() for t in fs.frame()) for _ in range(steps)]


def test_workload_constants_match_pages():
    g = json.load(open(os.path.join(GOLDEN, "pages_workload.json")))
    assert W.BLOCKS == g["blocks"] and W.PASSES == g["passes"]
    assert W.CALLS_PER_STEP == g["calls_per_step"] == g["blocks"] * g["passes"]
    assert W.PROD.shape.capacity == g["slots"] and W.PROD.shape.new_tokens == g["new_tokens"]
    assert W.RESET_PERIOD == g["reset_period_steps"]


@pytest.mark.parametrize("C,lengths", [
    (64, [16] * 10),
    (50, [7, 16, 16, 16, 3, 16, 16, 16]),
    (5788, [431] + [757] * 9),        # variable first forward, then steady frames
])
def test_slots_and_positions_follow_time_order(C, lengths):
    H, d = 1, 8
    rc = RingCache(H, d, C, max_new_tokens=max(lengths), mode="fp64")
    rng = np.random.default_rng(0)
    T = 0
    for step, n in enumerate(lengths):
        if step == 5:
            rc.rebase(rc.next_pos)        # positions reset to 0 in the middle
        rc.write(rng.standard_normal((n, H, d)), rng.standard_normal((n, H, d)))
        T += n
        assert rc.tokens == T
        assert rc.write_slot == T % C
        assert rc.n_valid == min(T, C)
        # walking the ring from the oldest slot gives consecutive positions
        order = rc.time_order()
        assert np.array_equal(order, np.arange(T - min(T, C), T) % C)
        p = rc.pos[order]
        assert np.all(np.diff(p) == 1)
        assert p[-1] == rc.next_pos - 1


def test_ring_equals_linear_read_time_rope_exact():
    """Ring + write-time RoPE (+ resets by delta rotation) == linear window + RoPE on
    every read, in exact arithmetic; the config wraps after 4 frames and resets
    every 3 steps."""
    frames = tiny_frames(10)
    s = W.TINY.shape
    rc = RingCache(s.heads, s.head_dim, s.capacity, mode="fp64")
    lc = LinearCache(s.heads, s.head_dim, s.capacity, mode="fp64")
    for step, (q, k, v) in enumerate(frames):
        if step > 0 and step % W.TINY.reset_period == 0:
            rc.rebase(rc.next_pos)
        rc.write(k, v)
        lc.write(k, v)
        assert rel(rc.attend(q), lc.attend(q)) < 1e-9


def test_ring_fp8_close_to_exact():
    """The FP8 ring stays within FP8 quantisation noise of the exact result, and the
    launch software's per-call re-quantisation lands in the same band."""
    frames = tiny_frames(10)
    s = W.TINY.shape
    rc = RingCache(s.heads, s.head_dim, s.capacity, max_position=s.max_position)
    ex = LinearCache(s.heads, s.head_dim, s.capacity, mode="fp64")
    rc.calibrate(frames[0][1], frames[0][2])
    lq = LinearCache(s.heads, s.head_dim, s.capacity, mode="fp8", scales=rc.scales())
    for step, (q, k, v) in enumerate(frames):
        if step > 0 and step % W.TINY.reset_period == 0:
            rc.rebase(rc.next_pos)
        rc.write(k, v)
        ex.write(k, v)
        lq.write(k, v)
        r = ex.attend(q)
        assert rel(rc.attend(q), r) < 0.15
        assert rel(lq.attend(q), r) < 0.15


def test_slot_order_positions_invalid_after_wrap():
    frames = tiny_frames(8)
    s = W.TINY.shape
    so = SlotOrderRing(s.heads, s.head_dim, s.capacity)
    lc = LinearCache(s.heads, s.head_dim, s.capacity, mode="fp64")
    T = 0
    for step, (q, k, v) in enumerate(frames):
        so.write(k, v)
        lc.write(k, v)
        T += k.shape[0]
        err = rel(so.attend(q), lc.attend(q))
        # slot order is time order until the ring wraps, and again whenever the
        # write slot comes back to 0 (T a multiple of C)
        if T <= s.capacity or T % s.capacity == 0:
            assert err < 1e-9, step
        else:
            assert err > 0.1, step


def test_delta_rotation_equals_rerotation_from_scratch():
    s = W.TINY.shape
    frames = tiny_frames(3)
    # exact arithmetic
    r64 = RingCache(s.heads, s.head_dim, s.capacity, mode="fp64")
    raw = []
    for _, k, v in frames:
        r64.write(k, v)
        raw.append(k)
    D = r64.next_pos
    r64.rebase(D)
    raw = np.concatenate(raw)                            # token t in slot t
    fresh = rope.rotate64(raw.astype(np.float64), np.arange(raw.shape[0]) - D, s.head_dim)
    assert np.max(np.abs(np.transpose(r64.k[:, :raw.shape[0]], (1, 0, 2)) - fresh)) < 1e-11
    assert np.array_equal(r64.pos[:raw.shape[0]], np.arange(raw.shape[0]) - D)
    # FP8: the code-domain rotation stays within two E4M3 steps (at the pair's
    # magnitude) of the exactly re-rotated key: one rounding before the
    # rotation, carried through it, and one after. Pairs whose norm reaches the
    # +-448 clamp are excluded, since saturation may cut them either way.
    r8 = RingCache(s.heads, s.head_dim, s.capacity, max_position=s.max_position)
    r8.calibrate(frames[0][1], frames[0][2])
    for _, k, v in frames:
        r8.write(k, v)
    r8.rebase(D)
    sc = r8.scale_k.astype(np.float64)[:, None, None]
    got = e4m3.decode(r8.k[:, :raw.shape[0]])
    ref = fresh.transpose(1, 0, 2) / sc                  # in code units
    pm = np.repeat(np.maximum(np.abs(ref[..., 0::2]), np.abs(ref[..., 1::2])), 2, axis=-1)
    norm = np.repeat(np.hypot(ref[..., 0::2], ref[..., 1::2]), 2, axis=-1)
    step = np.exp2(np.floor(np.log2(np.maximum(pm, 2.0 ** -6))) - 3)
    ok = norm <= 448.0
    assert ok.mean() > 0.9
    assert np.all(np.abs(got - ref)[ok] <= 2.0 * step[ok])


def test_attention_invariant_under_rebase():
    """A rebase changes positions, not attention: the same queries give the same output."""
    s = W.TINY.shape
    frames = tiny_frames(6)
    r64 = RingCache(s.heads, s.head_dim, s.capacity, mode="fp64")
    for _, k, v in frames:
        r64.write(k, v)
    q = frames[-1][0]
    before = r64.attend(q)
    r64.rebase(r64.next_pos - 3)
    assert rel(r64.attend(q), before) < 1e-10


def test_calibration_closed_form():
    s = W.TINY.shape
    q, k, v = tiny_frames(1)[0]
    rc = RingCache(s.heads, s.head_dim, s.capacity, max_position=s.max_position)
    rc.calibrate(k, v)
    c, sn = rope.cos_sin(np.arange(k.shape[0]), s.head_dim)
    kr = rope.rotate(k, c[:, None, :], sn[:, None, :])
    mk = max(abs(float(x)) for x in kr.ravel())
    mv = max(abs(float(x)) for x in v.ravel())
    assert rc.scale_k[0] == np.float32(mk / 448.0) and rc.inv_k[0] == np.float32(448.0 / mk)
    assert rc.scale_v[0] == np.float32(mv / 448.0) and rc.inv_v[0] == np.float32(448.0 / mv)
    # the calibrating frame itself never saturates: its absmax maps to at most 448
    rc.write(k, v)
    codes = rc.k[0, :k.shape[0]]
    assert np.max(np.abs(e4m3.decode(codes))) <= 448.0
    zero = RingCache(1, 4, 8)
    zero.calibrate(np.zeros((2, 1, 4), np.float32), np.zeros((2, 1, 4), np.float32))
    assert zero.scales().tolist() == [[1.0], [1.0], [1.0], [1.0]]


def test_write_bytes_are_scaled_rotated_codes():
    """Element check against the definition: code = E4M3(clamp(fl(rot(k) * inv)))."""
    s = W.TINY.shape
    frames = tiny_frames(5)
    rc = RingCache(s.heads, s.head_dim, s.capacity, max_position=s.max_position)
    rc.calibrate(frames[0][1], frames[0][2])
    for _, k, v in frames:
        rc.write(k, v)
    t = 4 * 16 + 5                         # a token of the fifth frame (wrapped)
    k = frames[4][1][5, 0]
    v = frames[4][2][5, 0]
    slot = t % s.capacity
    c, sn = rope.cos_sin([t], s.head_dim)
    for i in range(s.head_dim // 2):
        a, b = np.float32(k[2 * i]), np.float32(k[2 * i + 1])
        ar = np.float32(np.float32(a * c[0, i]) - np.float32(b * sn[0, i]))
        br = np.float32(np.float32(a * sn[0, i]) + np.float32(b * c[0, i]))
        for j, val in ((2 * i, ar), (2 * i + 1, br)):
            y = np.float32(val * rc.inv_k[0])
            assert rc.k[0, slot, j] == e4m3.encode(np.array([y]))[0]
    y = (v * rc.inv_v[0]).astype(np.float32)
    assert np.array_equal(rc.v[0, slot], e4m3.encode(y))
    assert rc.pos[slot] == t


def test_attention_independent_of_slot_order_and_heads():
    rng = np.random.default_rng(7)
    q = rng.standard_normal((5, 3, 16))
    k = rng.standard_normal((3, 40, 16))
    v = rng.standard_normal((3, 40, 16))
    o = softmax_attention(q, k, v)
    perm = rng.permutation(40)
    assert np.max(np.abs(softmax_attention(q, k[:, perm], v[:, perm]) - o)) < 1e-12
    k2 = k.copy()
    k2[1] += 5.0
    o2 = softmax_attention(q, k2, v)
    assert np.array_equal(o2[:, 0], o[:, 0]) and np.array_equal(o2[:, 2], o[:, 2])


def test_errors():
    rc = RingCache(2, 8, 16, max_new_tokens=8, max_position=40)
    x = np.zeros((4, 2, 8), np.float32)
    with pytest.raises(RuntimeError):
        rc.write(x, x)                       # before calibrate
    with pytest.raises(RuntimeError):
        rc.attend(x)                         # before any write
    rc.calibrate(x, x)
    with pytest.raises(ValueError):
        rc.write(np.zeros((9, 2, 8), np.float32), np.zeros((9, 2, 8), np.float32))
    for _ in range(10):
        rc.write(x, x)
    with pytest.raises(OverflowError):
        rc.write(x, x)                       # positions would reach max_position
    with pytest.raises(OverflowError):
        rc.rebase(rc.next_pos + 1)
    rc.rebase(rc.next_pos)
    assert rc.next_pos == 0 and rc.pos.min() == -16 and rc.pos.max() == -1
