"""Pins of the oracle's bfloat16 codec and of the ring's bf16 mode (the non-FP8
cache variant): torch's bfloat16 conversion, exact round trips, agreement of the
bf16 ring with the exact ring and with re-rotation from scratch."""
import numpy as np
import pytest
import torch

from oracle import bf16, rope
from oracle.cache import RingCache
from streaming_fp8_kv_amd import workloads as W

pytestmark = pytest.mark.cpu


def torch_bf16_bits(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_decode_matches_library_for_every_finite_pattern():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    finite = ((bits >> 7) & 0xFF) != 0xFF
    got = bf16.decode(bits[finite])
    ref = torch.from_numpy(bits[finite].view(np.int16)).view(torch.bfloat16).float().numpy()
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


def test_round_trip_of_every_finite_pattern():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    bits = bits[((bits >> 7) & 0xFF) != 0xFF]
    assert np.array_equal(bf16.encode(bf16.decode(bits)), bits)


@pytest.mark.parametrize("scale", [1e-40, 1e-30, 1e-3, 1.0, 100.0, 1e30])
def test_encode_matches_library_on_random_values(scale):
    x = (np.random.default_rng(1).standard_normal(200000) * scale).astype(np.float32)
    assert np.array_equal(bf16.encode(x), torch_bf16_bits(x))


def test_ties_round_to_even():
    # exact midpoints between neighbouring bf16 values, and one fp32 ulp to each side
    base = bf16.decode(np.arange(0x3F80, 0x4000, dtype=np.uint16))   # [1, 2)
    step = np.float32(2.0 ** -7)
    mids = (base + step / np.float32(2)).astype(np.float32)
    for x in (mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(4))):
        assert np.array_equal(bf16.encode(x), torch_bf16_bits(x))
    enc = bf16.encode(mids)
    assert np.all((enc & 1) == 0)                 # ties land on even patterns


def test_bf16_ring_stores_rounded_rotation_of_the_exact_keys():
    frames = [tuple(t.numpy() for t in W.FrameStream(W.TINY).frame()) for _ in range(6)]
    s = W.TINY.shape
    rb = RingCache(s.heads, s.head_dim, s.capacity, s.new_tokens, max_position=s.max_position, mode="bf16")
    ex = RingCache(s.heads, s.head_dim, s.capacity, s.new_tokens, max_position=s.max_position, mode="fp64")
    rb.calibrate(frames[0][1], frames[0][2])
    for q, k, v in frames:
        rb.write(k, v)
        ex.write(k, v)
    kb = bf16.decode(rb.k).astype(np.float64)
    # fp32 rotation then one bf16 rounding: within a bf16 half-ulp plus fp32 noise
    tol = np.abs(ex.k) * (2.0 ** -8 + 2.0 ** -21) + 1e-30
    assert np.all(np.abs(kb - ex.k) <= tol)
    assert np.array_equal(bf16.decode(rb.v).astype(np.float64), ex.v.astype(np.float32).astype(np.float64)) or \
        np.all(np.abs(bf16.decode(rb.v) - ex.v) <= np.abs(ex.v) * 2.0 ** -8)
    # attention in bf16 stays within bf16 noise of exact attention
    q = frames[-1][0]
    a, b = rb.attend(q), ex.attend(q)
    assert np.max(np.abs(a - b)) / np.max(np.abs(b)) < 2e-2


def test_bf16_rebase_equals_rerotation_from_scratch():
    s = W.TINY.shape
    frames = [tuple(t.numpy() for t in W.FrameStream(W.TINY).frame()) for _ in range(3)]
    rb = RingCache(s.heads, s.head_dim, s.capacity, s.new_tokens, max_position=s.max_position, mode="bf16")
    rb.calibrate(frames[0][1], frames[0][2])
    for _, k, v in frames:
        rb.write(k, v)
    delta = 29
    before_pos = rb.pos[:rb.n_valid].copy()
    rb.rebase(delta)
    got = bf16.decode(rb.k[:, :rb.n_valid]).astype(np.float64)
    # from scratch: every raw key rotated at its new position, rounded once
    raw = np.concatenate([f[1] for f in frames])                     # [T, H, d], token order = slot order
    c, s_ = rope.cos_sin(before_pos - delta, s.head_dim, s.rope_base)
    want = bf16.decode(bf16.encode(rope.rotate(raw, c[:, None, :], s_[:, None, :]))).astype(np.float64)
    want = np.transpose(want, (1, 0, 2))
    # two roundings (write, rebase) against one; the rotation mixes the two
    # elements of a pair, so each rounding error is bounded by a bf16 half-ulp
    # of the pair's norm
    norm = np.sqrt(want[..., 0::2] ** 2 + want[..., 1::2] ** 2)
    norm = np.repeat(norm, 2, axis=-1)
    assert np.all(np.abs(got - want) <= norm * 3 * 2.0 ** -8 + 1e-30)
    assert np.array_equal(rb.pos[:rb.n_valid], before_pos - delta)
