"""Pins for the oracle's MXFP8 query mode (CPU only).

The mode rounds each query row to MXFP8 along head_dim (E4M3 elements, one
UE8M0 power-of-two scale per 32 values by the OCP MX rule) before the
attention.  The checks below rebuild the E4M3 grid from its bit definition
and search it by brute force, instead of calling the oracle's scalar codecs.
"""

import math

import numpy as np
import pytest
import torch

from oracle import attention as A, layout as Lo


def _bf16(x):
    return (torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
            .view(torch.int16).numpy().view(np.uint16))


def _bf16_value(bits):
    return (np.asarray(bits, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)


# finite E4M3 magnitudes, code c = (E << 3) | m for c in 0 .. 126 (0x7F is NaN):
# E = 0 is subnormal, m * 2^-9; otherwise (1 + m / 8) * 2^(E - 7)
E4M3 = np.array([(c & 7) * 2.0 ** -9 if (c >> 3) == 0 else (1 + (c & 7) / 8) * 2.0 ** ((c >> 3) - 7)
                 for c in range(127)])


def _scale(amax):
    """OCP MX: X = 2^(floor(log2 amax) - 8) for E4M3 (largest exponent 8)."""
    m, e = math.frexp(amax)  # amax = m * 2^e, m in [0.5, 1)
    return 2.0 ** (e - 1 - 8)


def _brute_group(x):
    """Round a 32-value group to the nearest point of E4M3 * X, ties to the
    even code, magnitudes above 448 X clamped to 448 X."""
    amax = float(np.max(np.abs(x)))
    if amax == 0.0:
        return np.zeros_like(x)
    X = _scale(amax)
    out = np.empty_like(x)
    for i, v in enumerate(x):
        mag = min(abs(v) / X, 448.0)
        d = np.abs(E4M3 - mag)
        best = np.flatnonzero(d == d.min())
        c = best[0] if len(best) == 1 else [b for b in best if b % 2 == 0][0]
        out[i] = math.copysign(E4M3[c] * X, v) if E4M3[c] != 0 else 0.0
    return out


def _rows(rng, n, D=256):
    """bf16 rows with spread magnitudes, zero groups, and elements placed
    exactly on midpoints between grid points."""
    x = rng.standard_normal((n, D)) * np.exp2(rng.integers(-14, 6, size=(n, 1)))
    x[0, :32] = 0.0                                  # an all-zero group
    x[1, 32:64] *= 1e-30                             # a group far below 1
    g = x[2, :32]
    g[0] = 300.0                                     # X = 1 for this group
    g[1:9] = [1.0625, 1.1875, 17.0, 19.0, 0.5 + 2 ** -10, 2 ** -10, 3 * 2 ** -10, 460.0]  # midpoints, saturation
    return _bf16_value(_bf16(x)).reshape(n, D)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_query_rounding_equals_brute_force_nearest(seed):
    rng = np.random.default_rng(100 + seed)
    x = _rows(rng, 6)
    got = A.quantize_query_mxfp8(x)
    for r in range(x.shape[0]):
        for grp in range(x.shape[1] // 32):
            sl = slice(32 * grp, 32 * grp + 32)
            ref = _brute_group(x[r, sl])
            assert np.array_equal(got[r, sl], ref), (r, grp, got[r, sl][got[r, sl] != ref], ref[got[r, sl] != ref])


def test_midpoints_round_to_even_codes_and_saturation():
    x = np.zeros((1, 32))
    x[0, :6] = [300.0, 1.0625, 1.1875, 17.0, 19.0, 460.0]  # X = 2^0
    got = A.quantize_query_mxfp8(x)[0, :6]
    # 1.0625 lies between 1 (m = 0) and 1.125 (m = 1): even 1; 1.1875 between
    # 1.125 and 1.25: even 1.25; 17 between 16 and 18: 16; 19 between 18 and
    # 20: 20; 460 > 448: clamped
    assert got.tolist() == [288.0, 1.0, 1.25, 16.0, 20.0, 448.0]


def test_representable_query_is_unchanged():
    """Rows already on the grid (each group's largest magnitude in [256, 448]
    times a power of two, the rest E4M3 values at that scale) come back
    exactly, and the mode's attention is then the plain attention."""
    rng = np.random.default_rng(7)
    D, n = 256, 8
    codes = rng.integers(0, 127, size=(n, D))
    vals = E4M3[codes] * rng.choice([-1.0, 1.0], size=(n, D))
    big = rng.choice(np.flatnonzero((E4M3 >= 256) & (E4M3 <= 448)), size=(n, D // 32))
    vals[:, ::32] = E4M3[big]
    vals *= np.repeat(np.exp2(rng.integers(-20, 4, size=(n, D // 32))), 32, axis=1)
    assert np.array_equal(_bf16_value(_bf16(vals)), vals)  # representable in bf16 too
    assert np.array_equal(A.quantize_query_mxfp8(vals), vals)
    geo, pool, bt, lens = _small_cache()
    qb = _bf16(vals.reshape(2, 1, 4, D))
    o1, l1 = A.attention_ref(geo, pool, qb, bt, lens, 0.0625, 1, q_mxfp8=True)
    o0, l0 = A.attention_ref(geo, pool, qb, bt, lens, 0.0625, 1)
    assert np.array_equal(o1, o0) and np.array_equal(l1, l0)


def test_scale_rule_and_error_bounds():
    rng = np.random.default_rng(11)
    x = _rows(rng, 16)
    got = A.quantize_query_mxfp8(x)
    for r in range(x.shape[0]):
        for grp in range(x.shape[1] // 32):
            g, q = x[r, 32 * grp:32 * grp + 32], got[r, 32 * grp:32 * grp + 32]
            amax = np.abs(g).max()
            if amax == 0:
                assert np.all(q == 0)
                continue
            X = _scale(amax)
            assert 256 <= amax / X < 512
            assert np.all(np.abs(q) <= 448 * X)
            err = np.abs(q - g)
            normal = (np.abs(g) >= 2.0 ** -6 * X) & (np.abs(g) <= 448 * X)
            sub = np.abs(g) < 2.0 ** -6 * X
            sat = np.abs(g) > 448 * X
            assert np.all(err[normal] <= 2.0 ** -4 * np.abs(g[normal]))  # half a unit of 3 mantissa bits
            assert np.all(err[sub] <= 2.0 ** -10 * X)                    # half the subnormal step 2^-9 X
            assert np.all(err[sat] < 64 * X)
            assert np.all(np.sign(q[q != 0]) == np.sign(g[q != 0]))


def _small_cache():
    rng = np.random.default_rng(3)
    geo = Lo.Geometry(5, 256, 64, 2)
    lens = np.array([70, 9])
    bt = np.array([[0, 1], [2, 0]])
    pool = np.full(3 * geo.page_bytes, 0xFF, dtype=np.uint8)
    slots = np.concatenate([bt[b, np.arange(L) // 64] * 64 + np.arange(L) % 64 for b, L in enumerate(lens)])
    K = _bf16(rng.standard_normal((lens.sum(), 2, 256)))
    V = _bf16(rng.standard_normal((lens.sum(), 2, 256)))
    A.quantize_append(geo, pool, K, V, slots)
    return geo, pool, bt, lens


def test_mode_is_plain_attention_on_the_rounded_query():
    """The mode changes the query and nothing else: it equals the plain
    attention on the rounded query (representable in bf16: E4M3 values
    times a power of two), and differs from the plain attention on q."""
    geo, pool, bt, lens = _small_cache()
    rng = np.random.default_rng(5)
    qb = _bf16(rng.standard_normal((2, 1, 4, 256)))
    qx = A.quantize_query_mxfp8(_bf16_value(qb).reshape(qb.shape))
    assert np.array_equal(_bf16_value(_bf16(qx)).reshape(qx.shape), qx)
    o1, l1 = A.attention_ref(geo, pool, qb, bt, lens, 0.0625, 1, q_mxfp8=True)
    o2, l2 = A.attention_ref(geo, pool, _bf16(qx), bt, lens, 0.0625, 1)
    o0, _ = A.attention_ref(geo, pool, qb, bt, lens, 0.0625, 1)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    assert not np.array_equal(o1, o0)
    assert np.abs(o1 - o0).max() < 0.05  # 3-bit mantissas: a small change
