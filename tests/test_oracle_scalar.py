"""Pins for the oracle's scalar codecs (CPU only).

Each codec is checked against something other than its own formula:
library conversions (torch's float8_e4m3fn, NumPy's float16), brute-force
nearest-grid-point search, exhaustive round trips of every representable
value, and hand-constructed ties and saturation edges.
"""

import math

import numpy as np
import pytest
import torch

from oracle import scalar as S


def _e4m3_grid():
    """All finite non-negative E4M3FN values with their codes, built by
    enumerating sign-free bit patterns through torch's float8 type."""
    codes = torch.arange(0, 127, dtype=torch.int32).to(torch.uint8)
    vals = codes.view(torch.float8_e4m3fn).float().double().numpy()
    return np.arange(127), vals


def test_e4m3_decode_matches_torch_float8():
    codes = np.arange(256)
    ref = torch.from_numpy(codes.astype(np.uint8)).view(torch.float8_e4m3fn).float().double().numpy()
    got = S.e4m3_decode(codes)
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], got[ok])
    assert np.sum(np.isnan(got)) == 2  # 0x7F and 0xFF only
    assert got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9 and got[0x08] == 2.0 ** -6


def test_e4m3_round_trip_every_finite_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)])
    vals = S.e4m3_decode(codes).astype(np.float32)
    assert np.array_equal(S.e4m3_encode(vals), codes.astype(np.uint8))


def _brute_e4m3(x):
    """Nearest grid value by exhaustive search; ties -> even code; |x| >= 448 -> 448."""
    codes, grid = _e4m3_grid()
    out = []
    for v in np.asarray(x, dtype=np.float32).astype(np.float64):
        a = min(abs(v), 448.0)
        dist = np.abs(grid - a)
        best = np.flatnonzero(dist == dist.min())
        c = best[0] if len(best) == 1 else [b for b in best if b % 2 == 0][0]
        out.append(c | (0x80 if math.copysign(1.0, v) < 0 else 0))
    return np.array(out, dtype=np.uint8)


def _midpoints_e4m3():
    codes, grid = _e4m3_grid()
    xs = []
    for a, b in zip(grid[:-1], grid[1:]):
        m = np.float32((a + b) / 2)  # exact: grid values have <= 4 significant bits
        for v in (m, np.nextafter(m, np.float32(1e9)), np.nextafter(m, np.float32(-1e9)),
                  np.float32(a), np.float32(b)):
            xs += [v, -v]
    return np.array(xs, dtype=np.float32)


def test_e4m3_encode_ties_and_midpoints_brute_force():
    x = _midpoints_e4m3()
    assert np.array_equal(S.e4m3_encode(x), _brute_e4m3(x))


def test_e4m3_encode_random_brute_force_and_torch():
    rng = np.random.default_rng(7)
    x = np.concatenate([
        rng.standard_normal(4000) * 100,
        rng.standard_normal(2000) * 2.0 ** -8,      # subnormal range
        rng.uniform(-460, 460, 2000),
    ]).astype(np.float32)
    got = S.e4m3_encode(x)
    assert np.array_equal(got, _brute_e4m3(x))
    # torch's cast is IEEE RNE but turns values past the top midpoint into NaN:
    # compare on values clamped to the finite range
    xc = np.clip(x, -448, 448)
    ref = torch.from_numpy(xc).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(S.e4m3_encode(xc), ref)


def test_e4m3_saturation_and_signed_zero():
    x = np.array([448.0, 449.0, 464.0, 480.0, 1e6, 3.0e38, -500.0, -0.0, 0.0, 2.0 ** -11, -(2.0 ** -11)],
                 dtype=np.float32)
    assert list(S.e4m3_encode(x)) == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0x80, 0x00, 0x00, 0x80]


# ---------------------------------------------------------------- E2M1

def test_e2m1_table_and_round_trip():
    grid = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    for c in range(16):
        v = S.e2m1_decode(c)
        assert v == (-1 if c & 8 else 1) * grid[c & 7]
        assert S.e2m1_encode(np.float32(v)) == c or (c == 8 and v == 0)
    assert S.e2m1_encode(np.float32(-0.0)) == 8


def test_e2m1_ties_to_even_and_saturation():
    x = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.5, 100.0, 0.2499, 0.2501, 4.99, 5.01],
                 dtype=np.float32)
    want = [0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0, 6.0, 6.0, 0.0, 0.5, 4.0, 6.0]
    assert list(S.e2m1_decode(S.e2m1_encode(x))) == want
    assert list(S.e2m1_decode(S.e2m1_encode(-x))) == [-w for w in want]


def test_e2m1_random_brute_force():
    rng = np.random.default_rng(3)
    x = rng.uniform(-7, 7, 5000).astype(np.float32)
    grid = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    a = np.minimum(np.abs(x.astype(np.float64)), 6.0)
    d = np.abs(a[:, None] - grid[None, :])
    best = np.argmin(d, axis=1)  # no exact ties in continuous random data
    assert np.array_equal(np.abs(S.e2m1_decode(S.e2m1_encode(x))), grid[best])


# ---------------------------------------------------------------- UE8M0

def test_ue8m0_definition():
    rng = np.random.default_rng(5)
    amax = np.concatenate([np.exp(rng.uniform(-80, 80, 3000)), [1.0, 2.0, 255.9, 256.0, 448.0, 1e-30]]).astype(np.float32)
    b = S.ue8m0_from_amax(amax).astype(np.int64)
    for a, byte in zip(amax, b):
        m, e = math.frexp(float(a))  # a = m 2^e, m in [0.5, 1)
        assert byte == min(max(e - 1 - 8 + 127, 0), 254)
        if 0 < byte < 254:  # amax / X lies in [256, 512)
            assert 256.0 <= float(a) / 2.0 ** (byte - 127) < 512.0
    assert S.ue8m0_from_amax(np.float32(0)) == 0
    assert list(S.ue8m0_decode(np.array([127, 120, 0]))) == [1.0, 2.0 ** -7, 2.0 ** -127]


# ---------------------------------------------------------------- fp16

def test_f16_round_trip_all_finite_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    v = bits.view(np.float16)
    fin = np.isfinite(v)
    got = S.f32_to_f16_bits(v[fin].astype(np.float32))
    assert np.array_equal(got, bits[fin])


def test_f16_midpoints_ties_to_even():
    # midpoints between consecutive positive finite fp16 values, computed exactly
    bits = np.arange(0, 0x7BFF, dtype=np.uint16)
    lo = bits.view(np.float16).astype(np.float64)
    hi = (bits + 1).view(np.float16).astype(np.float64)
    mid = ((lo + hi) / 2).astype(np.float32)
    assert np.array_equal(mid.astype(np.float64), (lo + hi) / 2)  # representable in fp32
    got = S.f32_to_f16_bits(mid)
    want = np.where(bits % 2 == 0, bits, bits + 1).astype(np.uint16)
    assert np.array_equal(got, want)


def test_f16_scale_saturates():
    x = np.array([65504.0, 65519.0, 65520.0, 1e9, -1e9], dtype=np.float32)
    got = S.f16_bits_to_f64(S.f32_to_f16_sat_bits(x))
    assert list(got) == [65504.0, 65504.0, 65504.0, 65504.0, -65504.0]
    assert np.isinf(S.f16_bits_to_f64(S.f32_to_f16_bits(np.float32(65520.0))))


# ---------------------------------------------------------------- int8

def test_i8_ties_and_clamp():
    x = np.array([0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 126.5, 127.49, 127.5, 300.0, -300.0], dtype=np.float32)
    assert list(S.i8_encode(x)) == [0, 2, 2, 0, -2, -2, 126, 127, 127, 127, -127]


@pytest.mark.parametrize("broken", ["no_tie_even", "no_saturate"])
def test_planted_mistakes_are_caught(broken, monkeypatch):
    """A plausible slip in the E4M3 encoder must fail the brute-force pins."""
    def bad(x):
        x = np.asarray(x, dtype=np.float32)
        a = np.abs(x.astype(np.float64))
        if broken == "no_saturate":
            a = np.minimum(a, 1e4)  # forgets the clamp to 448
        else:
            a = np.minimum(a, 448.0)
        _, ex = np.frexp(np.where(a > 0, a, 1.0))
        e = np.where(a > 0, np.maximum(ex - 1.0, -6.0), -6.0)
        q = np.exp2(e - 3.0)
        if broken == "no_tie_even":
            m = np.floor(a / q + 0.5)  # ties away from zero
        else:
            m = np.rint(a / q)
        c = ((e + 6.0) * 8 + m).astype(np.int64) | np.where(np.signbit(x), 0x80, 0)
        return (c & 0xFF).astype(np.uint8)

    x = _midpoints_e4m3() if broken == "no_tie_even" else np.array([470.0, -480.0], dtype=np.float32)
    with pytest.raises(AssertionError):
        assert np.array_equal(bad(x), _brute_e4m3(x))
