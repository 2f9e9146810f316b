"""Scalar number formats: definitions of every code and scale type.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Every encoder takes float32 inputs (the value the quantizer divides out in
fp32) and rounds to nearest, ties to even, exactly as an IEEE conversion
would; the decoders return exact float64 values.  The element formats are
the ones the pages name: FP8 E4M3 (NInfer guide, FP8 entry; TokenSpeed
``fp8_e4m3``), 4-bit E2M1 with a UE4M3 scale byte (NInfer guide, NVFP4-G16
entry), UE8M0 block scales (TokenSpeed ``mxfp8`` entry), 8-bit integers with
group scales (NInfer guide, INT8-G64 entry) and FP16 scales / FP16 V
(NInfer guide, FP8 and BF16 entries).  The bit layouts are the public OCP
definitions; the pages only name the formats.
"""

import numpy as np

F16_MAX = 65504.0
E4M3_MAX = 448.0
E2M1_MAX = 6.0
I8_MAX = 127


# ----------------------------------------------------------------- bf16 / fp16

def bf16_bits_to_f32(bits):
    """bf16 bit patterns (uint16) -> float32 values (exact widening)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)


def f32_to_f16_bits(x):
    """IEEE float32 -> float16, round to nearest even, overflow -> +-inf.

    NumPy's float16 cast is the IEEE conversion (subnormals kept).  Used for
    the V plane of the BF16 format (NInfer guide, BF16 entry: V is written
    as FP16).  Pinned by the midpoint and exhaustive tests in
    ``tests/test_oracle_scalar.py``.
    """
    x = np.asarray(x, dtype=np.float32)
    with np.errstate(over="ignore"):
        return x.astype(np.float16).view(np.uint16)


def f32_to_f16_sat_bits(x):
    """float32 -> float16 bits, round to nearest even, saturating at +-65504.

    This is how every FP16 scale is stored (reading: a scale never becomes
    infinite).  Clamping first gives the same result as rounding then
    saturating, because 65504 is the largest finite value.
    """
    x = np.clip(np.asarray(x, dtype=np.float32), -F16_MAX, F16_MAX)
    return x.astype(np.float16).view(np.uint16)


def f16_bits_to_f64(bits):
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


# ----------------------------------------------------------------- E4M3 (FN)

def e4m3_decode(code):
    """E4M3FN code -> float64.  s.eeee.mmm, bias 7; E=0 is subnormal m*2^-9.

    0x7F / 0xFF are NaN (never written by the encoders).
    """
    c = np.asarray(code, dtype=np.int64)
    s = (c >> 7) & 1
    e = (c >> 3) & 15
    m = c & 7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return np.where(s == 1, -mag, mag)


def e4m3_encode(x):
    """float32 -> E4M3FN code, round to nearest even, saturate to +-448.

    Definition (OCP E4M3FN; the pages name the format only):
    a = |x| clamped to 448; e = max(floor(log2 a), -6) (the
    binade, with all values below 2^-6 sharing the subnormal quantum 2^-9);
    q = 2^(e-3) is the spacing of the grid in that binade; m = RNE(a / q).
    The code is then (e + 6) * 8 + m: for a normal value m lies in [8, 16]
    and (e + 6) * 8 + m = (biased exponent) * 8 + mantissa, a carry into the
    next binade included; for a subnormal value e = -6 and m in [0, 8].
    The sign bit is copied, so -0 encodes as 0x80.
    """
    x = np.asarray(x, dtype=np.float32).astype(np.float64)
    sign = np.signbit(x)
    a = np.minimum(np.abs(x), E4M3_MAX)
    # floor(log2 a) from frexp (a = mant * 2^ex, mant in [0.5, 1)): exact.
    mant, ex = np.frexp(np.where(a > 0, a, 1.0))
    e = np.where(a > 0, np.maximum(ex - 1.0, -6.0), -6.0)
    q = np.exp2(e - 3.0)
    m = np.rint(a / q)  # a / q is exact (power-of-two divisor); rint is RNE
    code = ((e + 6.0) * 8.0 + m).astype(np.int64)
    code = np.where(sign, code | 0x80, code)
    return code.astype(np.uint8)


def ue4m3_encode(x):
    """Unsigned E4M3 scale byte for x >= 0 (NVFP4-G16 group scale)."""
    x = np.asarray(x, dtype=np.float32)
    assert np.all(x >= 0)
    return e4m3_encode(x)


# ----------------------------------------------------------------- E2M1

E2M1_GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def e2m1_decode(code):
    """4-bit E2M1 code (s.ee.m, bias 1) -> float64; E=0 is subnormal m*0.5."""
    c = np.asarray(code, dtype=np.int64)
    mag = E2M1_GRID[c & 7]
    return np.where((c & 8) != 0, -mag, mag)


def e2m1_encode(x):
    """float32 -> E2M1 code, round to nearest even, saturate to +-6.

    Same construction as E4M3 with 1 mantissa bit: a = min(|x|, 6),
    e = max(floor(log2 a), 0), q = 2^(e-1), m = RNE(a / q) in [0, 4],
    code = 2e + m.  Sign copied into bit 3 (-0 -> 0x8).
    """
    x = np.asarray(x, dtype=np.float32).astype(np.float64)
    sign = np.signbit(x)
    a = np.minimum(np.abs(x), E2M1_MAX)
    mant, ex = np.frexp(np.where(a > 0, a, 1.0))
    e = np.where(a > 0, np.maximum(ex - 1.0, 0.0), 0.0)
    m = np.rint(a / np.exp2(e - 1.0))
    code = (2.0 * e + m).astype(np.int64)
    code = np.where(sign, code | 8, code)
    return code.astype(np.uint8)


# ----------------------------------------------------------------- UE8M0

def ue8m0_from_amax(amax, emax=8):
    """Shared exponent byte of an MX block (TokenSpeed ``mxfp8``: one UE8M0
    scale per 32 head_dim elements; ``mxfp4``: the 4-bit micro-scaling format).

    The page only names the scale type; the rule is the public OCP MX one:
    X = 2^(floor(log2 amax) - emax) with emax the element format's largest
    exponent (8 for E4M3, 2 for E2M1), stored biased by 127 and clamped to
    [0, 254].  amax = 0 gives byte 0.  floor(log2 amax) comes from frexp,
    which is exact.
    """
    a = np.asarray(amax, dtype=np.float32).astype(np.float64)
    mant, ex = np.frexp(np.where(a > 0, a, 1.0))
    b = np.clip(ex - 1 - emax + 127, 0, 254)
    return np.where(a > 0, b, 0).astype(np.uint8)


def ue8m0_decode(byte):
    return np.exp2(np.asarray(byte, dtype=np.float64) - 127.0)


# ----------------------------------------------------------------- INT8

def i8_encode(x):
    """float32 -> symmetric int8 code: RNE, clamped to [-127, 127]."""
    x = np.asarray(x, dtype=np.float32).astype(np.float64)
    return np.clip(np.rint(x), -I8_MAX, I8_MAX).astype(np.int8)
