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


# Quantiser pin: the scaled value is rounded to fp32 once before encoding
# ("Do It Once, at Write Time" stores each element as the E4M3 code of
# value x inverse scale; the reading fixes that product as one fp32 multiply).
# Each case is (x, inv, code), x and inv given as fp32 bit patterns. The exact
# product x * inv lies within a quarter of an fp32 ulp of a midpoint m between
# two adjacent E4M3 values, so fl32(x * inv) == m and ties-to-even picks the
# even code; the exact product lies on the other side of m, so a quantiser
# that encoded it without the fp32 rounding would pick the odd code.
#   x = m (1 + 2^-12), inv = 1 - 2^-12 + 2^-24: product m (1 + 2^-36), above m
#   x = m (1 + 2^-13), inv = 1 - 2^-13:         product m (1 - 2^-26), below m
_INV_ABOVE = 0x3F7FF001      # 1 - 2^-12 + 2^-24
_INV_BELOW = 0x3F7FF800      # 1 - 2^-13
QUANTISER_CASES = [
    # midpoint  x bits       inv bits    code (the even neighbour)
    (1.0625,    0x3F880880, _INV_ABOVE, 0x38),   # between 0x38 = 1.0 and 0x39 = 1.125
    (1.1875,    0x3F9804C0, _INV_BELOW, 0x3A),   # between 0x39 = 1.125 and 0x3A = 1.25
    (0.0029296875, 0x3B400600, _INV_BELOW, 0x02),  # subnormals 0x01 = 2^-9 and 0x02
    (0.0048828125, 0x3BA00A00, _INV_ABOVE, 0x02),  # subnormals 0x02 and 0x03
    (0.0146484375, 0x3C700780, _INV_BELOW, 0x08),  # largest subnormal 0x07 and 0x08 = 2^-6
    (0.033203125, 0x3D080880, _INV_ABOVE, 0x10),   # between 0x10 = 2^-5 and 0x11
    (21.0,      0x41A80A80, _INV_ABOVE, 0x5A),   # between 0x5A = 20 and 0x5B = 22
    (432.0,     0x43D806C0, _INV_BELOW, 0x7E),   # between 0x7D = 416 and 0x7E = 448
]


def _f32(bits):
    return np.array([bits], np.uint32).view(np.float32)


@pytest.mark.parametrize("mid,xb,ib,code", QUANTISER_CASES)
@pytest.mark.parametrize("sign", [1.0, -1.0])
def test_quantize_rounds_the_scaled_value_to_fp32_once(mid, xb, ib, code, sign):
    x, inv = _f32(xb) * np.float32(sign), _f32(ib)
    assert float((x * inv).astype(np.float32)[0]) == sign * mid     # fl32 lands on the midpoint
    want = code | (0x80 if sign < 0 else 0)
    assert int(e4m3.quantize(x, inv)[0]) == want


@pytest.mark.parametrize("mid,xb,ib,code", QUANTISER_CASES)
def test_quantiser_cases_separate_one_rounding_from_none(mid, xb, ib, code):
    """The exact product's nearest E4M3 value is the other neighbour of the
    midpoint: a quantiser without the fp32 rounding step fails the case above."""
    from fractions import Fraction
    p = Fraction(float(_f32(xb)[0])) * Fraction(float(_f32(ib)[0]))
    vals = [Fraction(float(v)) for v in e4m3.decode(np.arange(0, 0x7F))]
    nearest = min(range(len(vals)), key=lambda c: (abs(vals[c] - p), c % 2))
    assert p != Fraction(mid) and nearest != code
    assert {nearest, code} == {code, code + (1 if p > Fraction(mid) else -1)}
