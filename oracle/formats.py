"""KV-cache formats: how one (token, kv-head) row of K or V is encoded.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Each format pairs a K codec with a V codec (the NInfer guide's paged cache
keeps independent K and V encodings, and K8V4 is the fixed FP8-K /
NVFP4-V profile).  The codecs, from the NInfer guide's section on the five
formats unless noted:

=============  ======  =====================================================
codec          bits    per-row definition (x = the row, float32)
=============  ======  =====================================================
bf16           16      K of BF16: the input bf16 bits, unchanged
f16            16      V of BF16: IEEE float16 of the value
int8_g64       8       per 64 consecutive values: s = f16(amax / 127),
                       c = I8(x / s); K rotated first
e4m3_row       8       one FP16 scale per row: s = f16(amax / 448),
                       c = E4M3(x / s)
e2m1_g16       4       per 16 values: s = UE4M3(amax / 6), c = E2M1(x / s);
                       K and V rotated first (NVFP4-G16 entry).  Two-level
                       form: x is first divided by a per-tensor fp32 scale
                       g (IEEE fp32), so values decode to g * s * c; g = 1
                       is the single-level format (a reading: the pages
                       give NVFP4's 16-value groups and leave any level
                       above them open)
e4m3_mx32      8       per 32 values: one UE8M0 byte (OCP MX rule),
                       c = E4M3(x / 2^(byte-127)) (TokenSpeed ``mxfp8``)
e2m1_mx32      4       per 32 values: one UE8M0 byte (OCP MX rule with E2M1's
                       largest exponent 2), c = E2M1(x / 2^(byte-127)),
                       saturating; K and V rotated first (MXFP4 KV: the
                       pages' mxfp4 micro-scaling format applied to the cache,
                       rotated like their NVFP4 KV; a reading)
e4m3_tensor    8       c = E4M3(x / s) with one fp32 scale per tensor from
                       the caller (Qwen FP8-KV article: per-tensor
                       symmetric ``kv_cache_scheme``; TokenSpeed
                       ``fp8_e4m3`` "unit scale" is s = 1)
=============  ======  =====================================================

Groups run along head_dim inside one row (reading: "consecutive values"
of a token's vector).  Divisions are IEEE float32 and use the *stored*
scale; a scale that decodes to zero makes every code of its group zero.
Per-token byte counts follow and are pinned against the guide's table
(1024 / 528 / 516 / 288 / 402 B at head_dim 256) in
``tests/test_oracle_formats.py``.
"""

import numpy as np

from . import scalar as S
from .hadamard import fwht256_f32, unrotate_f64

# codec name -> (code bits, group size or None for whole-row/tensor, scale type)
CODECS = {
    "bf16": (16, None, None),
    "f16": (16, None, None),
    "int8_g64": (8, 64, "f16"),
    "e4m3_row": (8, "row", "f16"),
    "e2m1_g16": (4, 16, "ue4m3"),
    "e4m3_mx32": (8, 32, "ue8m0"),
    "e2m1_mx32": (4, 32, "ue8m0"),
    "e4m3_tensor": (8, None, None),
}
SCALE_BYTES = {None: 0, "f16": 2, "ue4m3": 1, "ue8m0": 1}

# format id (the C enum value) -> (name, K codec, V codec, K rotated, V rotated)
FORMATS = {
    0: ("BF16", "bf16", "f16", False, False),
    1: ("INT8_G64", "int8_g64", "int8_g64", True, False),
    2: ("FP8_ROW", "e4m3_row", "e4m3_row", False, False),
    3: ("NVFP4_G16", "e2m1_g16", "e2m1_g16", True, True),
    4: ("K8V4", "e4m3_row", "e2m1_g16", False, True),
    5: ("MXFP8", "e4m3_mx32", "e4m3_mx32", False, False),
    6: ("FP8_TENSOR", "e4m3_tensor", "e4m3_tensor", False, False),
    7: ("MXFP4", "e2m1_mx32", "e2m1_mx32", True, True),
}
FORMAT_IDS = {v[0]: k for k, v in FORMATS.items()}


def n_groups(codec, D):
    bits, group, stype = CODECS[codec]
    if stype is None:
        return 0
    return 1 if group == "row" else D // group


def row_bytes(codec, D):
    """Stored bytes of one row (codes plus its scales)."""
    bits, group, stype = CODECS[codec]
    return D * bits // 8 + n_groups(codec, D) * SCALE_BYTES[stype]


def token_bytes(fmt, D):
    """K+V bytes of one token of one kv head in one layer (the guide's
    per-token figure; page tables and alignment excluded)."""
    name, kc, vc, _, _ = FORMATS[fmt]
    return row_bytes(kc, D) + row_bytes(vc, D)


def _group_view(x, codec):
    D = x.shape[-1]
    bits, group, stype = CODECS[codec]
    g = D if group == "row" else group
    return x.reshape(x.shape[:-1] + (D // g, g))


def encode_rows(codec, rotated, rows, tensor_scale=1.0):
    """Encode rows (float32 [n, D]; for 'bf16' the uint16 bf16 bits).

    Returns (codes, scales): codes [n, D] (uint16 for 16-bit codecs, uint8
    otherwise, one 4-bit code per element for e2m1), scales [n, G] as raw
    stored bits (uint16 for f16 scales, uint8 for byte scales) or None.
    """
    if codec == "bf16":
        return np.asarray(rows, dtype=np.uint16).copy(), None
    x = np.asarray(rows, dtype=np.float32)
    if rotated:
        x = fwht256_f32(x)
    if codec == "f16":
        return S.f32_to_f16_bits(x), None
    if codec == "e4m3_tensor":
        s = np.float32(tensor_scale)
        assert s > 0
        return S.e4m3_encode((x / s).astype(np.float32)), None

    xg = _group_view(x, codec)
    amax = np.max(np.abs(xg), axis=-1)  # exact in float32
    if codec == "int8_g64":
        sbits = S.f32_to_f16_sat_bits((amax / np.float32(127.0)).astype(np.float32))
        s32 = sbits.view(np.float16).astype(np.float32)[..., None]
        with np.errstate(divide="ignore", invalid="ignore"):
            q = (xg / s32).astype(np.float32)
        c = np.where(s32 == 0, np.int8(0), S.i8_encode(np.where(s32 == 0, 0, q)))
        return c.reshape(x.shape).astype(np.int8).view(np.uint8), sbits
    if codec == "e4m3_row":
        sbits = S.f32_to_f16_sat_bits((amax / np.float32(448.0)).astype(np.float32))
        s32 = sbits.view(np.float16).astype(np.float32)[..., None]
        with np.errstate(divide="ignore", invalid="ignore"):
            q = (xg / s32).astype(np.float32)
        c = np.where(s32 == 0, np.uint8(0), S.e4m3_encode(np.where(s32 == 0, 0, q)))
        return c.reshape(x.shape).astype(np.uint8), sbits
    if codec == "e2m1_g16":
        g = np.float32(tensor_scale)
        assert g > 0
        x = (x / g).astype(np.float32)  # exact when g = 1
        xg = _group_view(x, codec)
        amax = np.max(np.abs(xg), axis=-1)
        sb = S.ue4m3_encode((amax / np.float32(6.0)).astype(np.float32))
        s32 = S.e4m3_decode(sb).astype(np.float32)[..., None]
        with np.errstate(divide="ignore", invalid="ignore"):
            q = (xg / s32).astype(np.float32)
        c = np.where(s32 == 0, np.uint8(0), S.e2m1_encode(np.where(s32 == 0, 0, q)))
        return c.reshape(x.shape).astype(np.uint8), sb
    if codec == "e2m1_mx32":
        sb = S.ue8m0_from_amax(amax, emax=2)
        X = S.ue8m0_decode(sb).astype(np.float32)[..., None]  # exact powers of two
        q = (xg / X).astype(np.float32)
        return S.e2m1_encode(q).reshape(x.shape).astype(np.uint8), sb
    if codec == "e4m3_mx32":
        sb = S.ue8m0_from_amax(amax)
        X = S.ue8m0_decode(sb).astype(np.float32)[..., None]  # exact powers of two
        q = (xg / X).astype(np.float32)
        return S.e4m3_encode(q).reshape(x.shape), sb
    raise ValueError(codec)


def decode_rows(codec, rotated, codes, scales, tensor_scale=1.0, stored_domain=False):
    """Exact float64 value of each stored element.

    Stored domain: dec(code) * dec(scale of its group).  Unless
    ``stored_domain`` is set, rotated planes are then mapped back with the
    float64 inverse rotation H y / 16.
    """
    codes = np.asarray(codes)
    if codec == "bf16":
        v = S.bf16_bits_to_f32(codes).astype(np.float64)
    elif codec == "f16":
        v = S.f16_bits_to_f64(codes)
    elif codec == "e4m3_tensor":
        v = S.e4m3_decode(codes) * float(np.float32(tensor_scale))
    else:
        bits, group, stype = CODECS[codec]
        if codec == "int8_g64":
            c = codes.astype(np.uint8).view(np.int8).astype(np.float64)
        elif codec in ("e2m1_g16", "e2m1_mx32"):
            c = S.e2m1_decode(codes)
        else:
            c = S.e4m3_decode(codes)
        if stype == "f16":
            s = S.f16_bits_to_f64(scales)
        elif stype == "ue4m3":
            s = S.e4m3_decode(scales)
        else:
            s = S.ue8m0_decode(scales)
        cg = _group_view(c, codec)
        v = (cg * s[..., None]).reshape(c.shape)
        if codec == "e2m1_g16":
            v = v * float(np.float32(tensor_scale))  # the two-level form's per-tensor scale
    if rotated and not stored_domain:
        v = unrotate_f64(v)
    return v
