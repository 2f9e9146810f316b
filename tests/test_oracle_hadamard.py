"""Pins for the oracle's 256-point Hadamard rotation (CPU only)."""

import numpy as np
import pytest
import scipy.linalg

from oracle import hadamard as Hd


def test_matrix_is_sylvester_hadamard():
    H = Hd.hadamard_matrix(256)
    assert np.array_equal(H, scipy.linalg.hadamard(256).astype(np.float64))
    assert np.array_equal(H @ H.T, 256.0 * np.eye(256))
    assert np.array_equal(H, H.T)


def test_fwht_of_unit_vectors_is_a_column():
    H = Hd.hadamard_matrix(256)
    E = np.eye(256, dtype=np.float32)
    R = Hd.fwht256_f32(E)  # row j is R(e_j)
    assert np.array_equal(R.astype(np.float64), H.T / 16.0)


def test_fwht_exact_on_small_integers():
    rng = np.random.default_rng(11)
    x = rng.integers(-(2 ** 15), 2 ** 15 + 1, size=(64, 256)).astype(np.float32)
    H = Hd.hadamard_matrix(256)
    # every partial sum is an integer below 2^23, so no rounding happens
    assert np.array_equal(Hd.fwht256_f32(x).astype(np.float64), x.astype(np.float64) @ H.T / 16.0)


def test_fwht_float32_error_bound():
    rng = np.random.default_rng(12)
    x = (rng.standard_normal((256, 256)) * np.exp(rng.uniform(-5, 5, (256, 1)))).astype(np.float32)
    H = Hd.hadamard_matrix(256)
    exact = x.astype(np.float64) @ H.T / 16.0
    u = 2.0 ** -24
    gamma8 = 8 * u / (1 - 8 * u)  # depth-8 butterfly tree
    bound = gamma8 * np.abs(x.astype(np.float64)).sum(axis=1) / 16.0
    err = np.abs(Hd.fwht256_f32(x).astype(np.float64) - exact).max(axis=1)
    assert np.all(err <= bound)
    # and it is not exact in general: float32 rounding does happen
    assert np.any(err > 0)


def test_parseval_and_involution():
    rng = np.random.default_rng(13)
    x = rng.standard_normal((8, 256))
    y = Hd.fwht256_f32(x.astype(np.float32)).astype(np.float64)
    assert np.allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-6)
    assert np.allclose(Hd.unrotate_f64(y), x.astype(np.float32), atol=1e-5)


def test_fwht_fixed_stage_order_matters():
    """The butterfly order is part of the format: a different order gives a
    different float32 result for some inputs (so a GPU using another order
    would be caught by the bit-exact codec tests)."""
    rng = np.random.default_rng(14)
    x = (rng.standard_normal((512, 256)) * 1000).astype(np.float32)

    def reversed_order(v):
        y = v.copy()
        h = 128
        while h >= 1:
            w = y.reshape(y.shape[:-1] + (256 // (2 * h), 2, h))
            a, b = w[..., 0, :], w[..., 1, :]
            y = np.stack([(a + b).astype(np.float32), (a - b).astype(np.float32)], axis=-2).reshape(y.shape)
            h //= 2
        return (y * np.float32(0.0625)).astype(np.float32)

    assert not np.array_equal(reversed_order(x), Hd.fwht256_f32(x))


@pytest.mark.parametrize("broken", ["skip_stage", "wrong_scale"])
def test_planted_mistakes_are_caught(broken):
    def bad(v):
        y = v.copy()
        h = 1
        while h < 256:
            if not (broken == "skip_stage" and h == 32):
                w = y.reshape(y.shape[:-1] + (256 // (2 * h), 2, h))
                a, b = w[..., 0, :], w[..., 1, :]
                y = np.stack([(a + b), (a - b)], axis=-2).reshape(y.shape).astype(np.float32)
            h *= 2
        return y * np.float32(1 / 256 if broken == "wrong_scale" else 1 / 16)

    E = np.eye(256, dtype=np.float32)
    assert not np.array_equal(bad(E).astype(np.float64), Hd.hadamard_matrix(256).T / 16.0)
