"""The 256-point normalized Hadamard rotation.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The NInfer guide applies a normalized 256-dimensional Hadamard transform to
K before INT8-G64 quantization, and to both K and V before NVFP4-G16
quantization (section on the five formats, INT8 and NVFP4 entries).  It
states neither the row order nor the arithmetic.  Readings taken:

* order: Sylvester ("natural") order, H[i, j] = (-1)^popcount(i & j), the
  matrix ``scipy.linalg.hadamard(256)`` returns;
* normalization: y = H x / 16, which makes the transform orthonormal
  (H H^T = 256 I), so its inverse is itself;
* arithmetic on the write path: the fixed radix-2 butterfly order of
  :func:`fwht256_f32`, every add/sub rounded once to float32, then an exact
  scaling by 2^-4.  The encoder's output therefore depends on float32
  rounding in a reproducible way, which the GPU must match bit for bit.

The read path (un-rotating decoded values) uses the exact float64 matrix.
"""

import numpy as np


def hadamard_matrix(n=256):
    """Sylvester Hadamard matrix as float64, built from the popcount rule."""
    i = np.arange(n)[:, None]
    j = np.arange(n)[None, :]
    ij = i & j
    pc = np.zeros_like(ij)
    for bit in range(int(np.log2(n)) + 1):
        pc += (ij >> bit) & 1
    return np.where(pc % 2 == 0, 1.0, -1.0)


def fwht256_f32(x):
    """y = H x / 16 over the last axis (length 256) in float32.

    For h = 1, 2, 4, ..., 128 in that order, every pair (i, i + h) with bit h
    of i clear becomes (y_i + y_{i+h}, y_i - y_{i+h}); each sum or difference
    is one float32 rounding (NumPy float32 arithmetic is IEEE).  Finally the
    vector is multiplied by 2^-4, which is exact.
    Pinned by: R(e_j) = H[:, j] / 16 exactly; exactness on small integers;
    the float32 error bound against the float64 product; Parseval.
    """
    y = np.array(x, dtype=np.float32, copy=True)
    assert y.shape[-1] == 256
    lead = y.shape[:-1]
    h = 1
    while h < 256:
        v = y.reshape(lead + (256 // (2 * h), 2, h))
        a = v[..., 0, :]
        b = v[..., 1, :]
        s = (a + b).astype(np.float32)
        d = (a - b).astype(np.float32)
        y = np.stack([s, d], axis=-2).reshape(lead + (256,))
        h *= 2
    return (y * np.float32(0.0625)).astype(np.float32)


def unrotate_f64(y):
    """Inverse rotation in float64: x = H y / 16 (H is symmetric, H H = 256 I)."""
    return np.asarray(y, dtype=np.float64) @ (hadamard_matrix(256) / 16.0)
