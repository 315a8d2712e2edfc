"""Pins of the oracle's OCP E4M3FN codec against the format's definition and a library routine."""
import numpy as np
import pytest
import torch

from oracle import e4m3

pytestmark = pytest.mark.cpu


def _torch_decode_all():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def _torch_encode(x):
    t = torch.from_numpy(np.clip(np.asarray(x, np.float32), -448, 448))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_decode_matches_library_for_all_codes():
    ours = e4m3.decode(np.arange(256))
    lib = _torch_decode_all()
    nan = np.isnan(lib)
    assert np.array_equal(nan, np.isnan(ours))
    assert set(np.nonzero(nan)[0].tolist()) == {0x7F, 0xFF}
    assert np.array_equal(ours[~nan], lib[~nan])


def test_decode_landmarks():
    d = e4m3.decode(np.array([0x00, 0x80, 0x01, 0x07, 0x08, 0x38, 0x7E, 0xFE]))
    assert d[0] == 0.0 and d[1] == 0.0 and np.signbit(d[1])
    assert d[2] == 2.0 ** -9                 # smallest subnormal
    assert d[3] == 7 * 2.0 ** -9             # largest subnormal
    assert d[4] == 2.0 ** -6                 # smallest normal
    assert d[5] == 1.0
    assert d[6] == 448.0 and d[7] == -448.0  # largest finite


def test_round_trip_every_finite_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = e4m3.decode(codes).astype(np.float32)
    assert np.array_equal(e4m3.encode(vals), codes)


def test_midpoints_round_to_even_and_neighbours_to_nearest():
    pos_codes = np.arange(0, 0x7F)                     # 0 .. 0x7E
    vals = e4m3.decode(pos_codes)
    for sign in (1.0, -1.0):
        for c in range(0x7E):
            lo, hi = vals[c], vals[c + 1]
            mid = np.float32((lo + hi) / 2)
            assert float(mid) == (lo + hi) / 2          # exact in fp32
            even = c if c % 2 == 0 else c + 1
            below = np.nextafter(mid, np.float32(0))
            above = np.nextafter(mid, np.float32(np.inf))
            sbit = 0x80 if sign < 0 else 0
            got = e4m3.encode(np.array([mid, below, above], np.float32) * np.float32(sign))
            assert got[0] == (even | sbit), (c, sign)
            assert got[1] == (c | sbit) or (c == 0 and sign < 0 and got[1] == 0x80)
            assert got[2] == ((c + 1) | sbit)


def _brute_nearest(x):
    """Nearest finite code by exhaustive search; ties to the even code."""
    cand = np.arange(0, 0x7F)
    cv = e4m3.decode(cand)
    out = np.empty(x.shape, dtype=np.uint8)
    for i, v in enumerate(np.clip(x.astype(np.float64), -448, 448)):
        dist = np.abs(np.abs(v) - cv)
        best = np.nonzero(dist == dist.min())[0]
        c = best[0] if len(best) == 1 else [b for b in best if b % 2 == 0][0]
        out[i] = c | (0x80 if np.signbit(v) else 0)
    return out


def test_brute_force_nearest_on_random_sample():
    rng = np.random.default_rng(11)
    mag = np.exp2(rng.uniform(-12, 9.2, size=20000)).astype(np.float32)
    x = (mag * rng.choice([-1, 1], size=mag.size)).astype(np.float32)
    assert np.array_equal(e4m3.encode(x), _brute_nearest(x))


@pytest.mark.parametrize("lo,hi", [(2.0 ** -8, 2.0 ** -5), (256.0, 448.0), (0.5, 2.0)])
def test_exhaustive_fp32_ranges_match_library(lo, hi):
    a = np.array([lo], np.float32).view(np.uint32)[0]
    b = np.array([hi], np.float32).view(np.uint32)[0]
    x = np.arange(a, b + 1, dtype=np.uint32).view(np.float32)
    assert np.array_equal(e4m3.encode(x), _torch_encode(x))
    assert np.array_equal(e4m3.encode(-x), _torch_encode(-x))


def test_random_fp32_match_library():
    rng = np.random.default_rng(5)
    x = (rng.standard_normal(2_000_000) * np.exp2(rng.uniform(-14, 10, 2_000_000))).astype(np.float32)
    assert np.array_equal(e4m3.encode(x), _torch_encode(x))


def test_saturation_and_signed_zero():
    x = np.array([448.0, 449.0, 464.0, 480.0, 1e30, -1e30, 0.0, -0.0, -1e-30], np.float32)
    assert e4m3.encode(x).tolist() == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0x00, 0x80, 0x80]


def test_quantize_rounds_scaled_value_once():
    x = np.array([1.0, 3.0, -7.5], np.float32)
    inv = np.float32(1.0 / 3.0)
    y = (x * inv).astype(np.float32)
    assert np.array_equal(e4m3.quantize(x, inv), e4m3.encode(y))
