"""Pins for the oracle's KV formats and page layout (CPU only).

Byte counts are pinned to the tables the pages print (tests/golden); each
codec to exact round trips of values on its grid, to its rounding error
bound, and to the grouping/rotation facts the guide states.
"""

import os

import numpy as np
import pytest

from oracle import formats as F, layout as Lo, scalar as S, hadamard as Hd

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_rows(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


def test_bytes_per_token_match_the_guide_table():
    rows = _golden_rows("kv_bytes_per_token.txt")
    assert len(rows) == 5
    for name, nbytes, pct in rows:
        fmt = F.FORMAT_IDS[name]
        assert F.token_bytes(fmt, 256) == int(nbytes)
        # the printed share of BF16 ("about N%"): the exact share truncated
        # to whole percent (528 B is 51.6%, printed as about 51%)
        assert int(100 * F.token_bytes(fmt, 256) / 1024) == int(pct)
    # "close to 3.5x the context" for NVFP4
    assert round(1024 / F.token_bytes(F.FORMAT_IDS["NVFP4_G16"], 256), 1) in (3.5, 3.6)


def test_kv_cache_dtype_ratios_match_tokenspeed_table():
    rows = {r[0]: float(r[2]) for r in _golden_rows("kv_cache_dtype_ratios.txt")}
    for D in (128, 256):
        bf16 = F.token_bytes(F.FORMAT_IDS["BF16"], D)
        fp8 = F.token_bytes(F.FORMAT_IDS["FP8_TENSOR"], D) / bf16
        mx = F.token_bytes(F.FORMAT_IDS["MXFP8"], D) / bf16
        assert fp8 == rows["fp8_e4m3"]
        # printed 0.5x leaves out the scale bytes: 1 byte per 32 codes
        assert mx == pytest.approx(rows["mxfp8"] * (1 + 1 / 32))


def test_m_kv_formula_for_bf16_pool():
    """llama.cpp FP8-KV article: M_KV = 2 B L H_kv S d_head elements over L
    layers; at 2 bytes per element a full BF16 pool for one layer is that."""
    B, layers, H_kv, S_, d = 3, 1, 4, 256, 256
    geo = Lo.Geometry(F.FORMAT_IDS["BF16"], d, 64, H_kv)
    pages = B * S_ // 64
    assert pages * geo.page_bytes == 2 * B * layers * H_kv * S_ * d * 2


def test_mxfp4_bytes_per_token():
    """E2M1 codes plus one UE8M0 byte per 32 values, K and V: 2 (128 + 8) =
    272 B per token and kv head at head_dim 256, below NVFP4's 288."""
    assert F.token_bytes(F.FORMAT_IDS["MXFP4"], 256) == 272
    assert F.token_bytes(F.FORMAT_IDS["MXFP4"], 256) < F.token_bytes(F.FORMAT_IDS["NVFP4_G16"], 256)


@pytest.mark.parametrize("fmt", range(8))
@pytest.mark.parametrize("P", [64, 128])
def test_page_is_exactly_per_token_bytes(fmt, P):
    D = 128 if fmt == 5 else 256
    geo = Lo.Geometry(fmt, D, P, 3)
    assert geo.page_bytes == 3 * P * F.token_bytes(fmt, D)
    assert all(o % 128 == 0 for o in geo.off)


def _grid_values(codec, rng, n, D):
    """Rows whose values lie exactly on codec grid x scale, with one element
    per group at the group maximum, so encoding must reproduce them."""
    bits, group, stype = F.CODECS[codec]
    g = D if group == "row" else group
    if codec == "int8_g64":
        c = rng.integers(-127, 128, (n, D)).astype(np.float64)
        qmax = 127.0
        s = S.f16_bits_to_f64(S.f32_to_f16_sat_bits(np.exp(rng.uniform(-8, 3, (n, D // g))).astype(np.float32)))
    elif codec == "e4m3_row":
        c = S.e4m3_decode(rng.integers(0, 127, (n, D))) * rng.choice([-1, 1], (n, D))
        qmax = 448.0
        s = S.f16_bits_to_f64(S.f32_to_f16_sat_bits(np.exp(rng.uniform(-8, 3, (n, 1))).astype(np.float32)))
    elif codec == "e2m1_g16":
        c = S.e2m1_decode(rng.integers(0, 16, (n, D)))
        qmax = 6.0
        s = S.e4m3_decode(rng.integers(8, 100, (n, D // g)))
    elif codec == "e2m1_mx32":
        c = S.e2m1_decode(rng.integers(0, 16, (n, D)))
        s = np.exp2(rng.integers(-20, 10, (n, D // g)).astype(np.float64))
        cg = c.reshape(n, D // g, g)
        cg[..., 0] = rng.choice([4.0, 6.0], (n, D // g))  # amax / X in [4, 8): the exponent the MX rule picks
        return (cg * s[..., None]).reshape(n, D).astype(np.float32), c, s
    else:  # e4m3_mx32
        c = S.e4m3_decode(rng.integers(0, 127, (n, D))) * rng.choice([-1, 1], (n, D))
        s = np.exp2(rng.integers(-20, 10, (n, D // g)).astype(np.float64))
        cg = c.reshape(n, D // g, g)
        cg[..., 0] = 256.0  # amax / X = 256 exactly: the top binade the MX rule picks
        return (cg * s[..., None]).reshape(n, D).astype(np.float32), c, s
    cg = c.reshape(n, D // g, g)
    cg[..., 0] = qmax
    return (cg * s[..., None]).reshape(n, D).astype(np.float32), c, s


@pytest.mark.parametrize("codec", ["int8_g64", "e4m3_row", "e2m1_g16", "e4m3_mx32", "e2m1_mx32"])
def test_round_trip_of_representable_rows(codec):
    rng = np.random.default_rng(21)
    x, c, s = _grid_values(codec, rng, 50, 256)
    assert np.array_equal(x.astype(np.float64).reshape(c.shape[0], -1),
                          (c.reshape(c.shape[0], s.shape[1], -1) * s[..., None]).reshape(c.shape[0], -1))
    codes, scales = F.encode_rows(codec, False, x)
    back = F.decode_rows(codec, False, codes, scales, stored_domain=True)
    assert np.array_equal(back, x.astype(np.float64))


@pytest.mark.parametrize("codec", ["int8_g64", "e4m3_row", "e2m1_g16", "e4m3_mx32", "e2m1_mx32", "e4m3_tensor",
                                   "f16"])
def test_error_bound_half_a_grid_step(codec):
    rng = np.random.default_rng(22)
    x = (rng.standard_normal((200, 256)) * np.exp(rng.uniform(-3, 3, (200, 1)))).astype(np.float32)
    codes, scales = F.encode_rows(codec, False, x, tensor_scale=0.05)
    xh = F.decode_rows(codec, False, codes, scales, tensor_scale=0.05, stored_domain=True)
    err = np.abs(xh - x.astype(np.float64))
    bits, group, stype = F.CODECS[codec]
    if codec == "f16":
        assert np.all(err <= np.abs(x) * 2.0 ** -11 + 2.0 ** -25)
        return
    if codec == "e4m3_tensor":
        rel, sub = 2.0 ** -4, 2.0 ** -10 * 0.05
        assert np.all((err <= np.abs(x) * rel + sub) | (np.abs(x) > 448 * 0.05))
        return
    g = 256 if group == "row" else group
    xg = np.abs(x.astype(np.float64)).reshape(200, 256 // g, g)
    amax = xg.max(axis=-1, keepdims=True)
    eg = err.reshape(200, 256 // g, g)
    if codec == "int8_g64":
        sc = S.f16_bits_to_f64(scales)[..., None]
        assert np.all(eg <= 0.5 * sc * (1 + 1e-6) + amax * 2.0 ** -11)
    elif codec == "e2m1_g16":
        sc = S.e4m3_decode(scales)[..., None]
        step = np.where(xg / sc < 2, 0.5, np.where(xg / sc < 4, 1.0, 2.0)) * sc
        assert np.all(eg <= 0.5 * step + amax * 2.0 ** -4)  # scale rounding may clip the top
    elif codec == "e2m1_mx32":  # amax / X in [4, 8): the grid step is X/2, X or 2X; above 6 X saturates
        X = S.ue8m0_decode(scales)[..., None]
        r = xg / X
        assert np.all((r[..., :].max(axis=-1) >= 4) & (r.max(axis=-1) < 8))
        step = np.where(r < 2, 0.5, np.where(r < 4, 1.0, 2.0)) * X
        clip = np.maximum(xg - 6.0 * X, 0.0)
        assert np.all(eg <= 0.5 * step + clip)
        assert np.any(clip > 0)
    elif codec == "e4m3_row":  # 3 mantissa bits; scale rounding clips at most amax 2^-11
        assert np.all(eg <= xg * 2.0 ** -4 + amax * 2.0 ** -9)
    else:  # MX: amax / X lies in [256, 512), so values above 448 X saturate
        X = S.ue8m0_decode(scales)[..., None]
        clip = np.maximum(xg - 448.0 * X, 0.0)
        assert np.all(eg <= xg * 2.0 ** -4 + X * 2.0 ** -10 + clip)
        assert np.any(clip > 0)


def test_groups_run_along_head_dim():
    """One large element raises only its own group's scale."""
    x = np.ones((1, 256), dtype=np.float32)
    x[0, 64 * 2 + 5] = 100.0
    _, s8 = F.encode_rows("int8_g64", False, x)
    sv = S.f16_bits_to_f64(s8)[0]
    assert np.argmax(sv) == 2 and np.sum(sv > sv.min()) == 1
    x = np.ones((1, 256), dtype=np.float32)
    x[0, 16 * 9 + 3] = 50.0
    _, s4 = F.encode_rows("e2m1_g16", False, x)
    assert np.argmax(S.e4m3_decode(s4[0])) == 9
    _, smx = F.encode_rows("e4m3_mx32", False, x)
    assert np.argmax(smx[0]) == (16 * 9 + 3) // 32


def test_zero_rows_give_zero_codes_and_scales():
    z = np.zeros((2, 256), dtype=np.float32)
    for codec in ("int8_g64", "e4m3_row", "e2m1_g16", "e4m3_mx32", "e4m3_tensor"):
        c, s = F.encode_rows(codec, codec == "e2m1_g16", z)
        assert not np.any(c)
        if s is not None:
            assert not np.any(s)


def test_rotation_is_applied_where_the_guide_says():
    """INT8: K rotated, V not; NVFP4: both; K8V4 keeps each half's rule."""
    assert [F.FORMATS[f][3:] for f in range(7)] == [
        (False, False), (True, False), (False, False), (True, True), (False, True), (False, False), (False, False)]
    # a unit spike is spread over all 256 stored values by the rotation
    x = np.zeros((1, 256), dtype=np.float32)
    x[0, 7] = 3.0
    c_rot, s_rot = F.encode_rows("e2m1_g16", True, x)
    stored = F.decode_rows("e2m1_g16", True, c_rot, s_rot, stored_domain=True)
    assert np.all(np.abs(stored) == 3.0 / 16)  # H[:, 7] / 16 * 3 is on the grid exactly
    back = F.decode_rows("e2m1_g16", True, c_rot, s_rot)
    assert np.allclose(back, x, atol=1e-12)


def test_k8v4_halves_equal_their_parent_formats():
    rng = np.random.default_rng(23)
    x = rng.standard_normal((8, 256)).astype(np.float32)
    name, kc, vc, kr, vr = F.FORMATS[F.FORMAT_IDS["K8V4"]]
    assert (kc, kr) == (F.FORMATS[2][1], F.FORMATS[2][3])
    assert (vc, vr) == (F.FORMATS[3][2], F.FORMATS[3][4])


def test_fp8_tensor_unit_scale_is_plain_e4m3():
    rng = np.random.default_rng(24)
    x = (rng.standard_normal((4, 256)) * 50).astype(np.float32)
    c, _ = F.encode_rows("e4m3_tensor", False, x, tensor_scale=1.0)
    assert np.array_equal(c, S.e4m3_encode(x))


# ------------------------------------------------- two-level NVFP4 (fp32 per-tensor scale)

@pytest.mark.parametrize("rotated", [False, True])
def test_two_level_nvfp4_power_of_two_scale_is_an_exact_rescaling(rotated):
    """Dividing by a global scale 2^-5 first is the same as encoding x * 2^5
    with no global scale: same code and block-scale bytes (a misplaced scale,
    say applied after the block scale, or multiplied, breaks this)."""
    rng = np.random.default_rng(31)
    x = (rng.standard_normal((16, 256)) * 0.05).astype(np.float32)
    c2, s2 = F.encode_rows("e2m1_g16", rotated, x, tensor_scale=2.0 ** -5)
    c1, s1 = F.encode_rows("e2m1_g16", rotated, (x * np.float32(32.0)).astype(np.float32), tensor_scale=1.0)
    assert np.array_equal(c2, c1) and np.array_equal(s2, s1)
    # and the decoded values carry the global scale back
    v2 = F.decode_rows("e2m1_g16", rotated, c2, s2, tensor_scale=2.0 ** -5)
    v1 = F.decode_rows("e2m1_g16", rotated, c1, s1, tensor_scale=1.0)
    assert np.allclose(v2, v1 / 32.0, rtol=0, atol=1e-12)


def test_two_level_nvfp4_round_trip_with_a_non_power_of_two_scale():
    """x = g * s_b * c built from codes, block scales (each group holding a
    +-6 code, so amax / 6 = s_b) and g = 3: encoding with g and decoding give
    x back exactly."""
    rng = np.random.default_rng(32)
    n, D, g = 8, 256, np.float32(3.0)
    c = S.e2m1_decode(rng.integers(0, 16, (n, D)))
    c = c.reshape(n, D // 16, 16)
    c[:, :, 0] = np.where(rng.integers(0, 2, (n, D // 16)) > 0, 6.0, -6.0)
    sb = S.e4m3_decode(rng.integers(0x08, 0x60, (n, D // 16)).astype(np.uint8))
    x = (g * sb[..., None] * c).reshape(n, D).astype(np.float32)
    assert np.array_equal(x.astype(np.float64), (3.0 * sb[..., None] * c).reshape(n, D))  # exact in fp32
    codes, scales = F.encode_rows("e2m1_g16", False, x, tensor_scale=float(g))
    back = F.decode_rows("e2m1_g16", False, codes, scales, tensor_scale=float(g))
    assert np.array_equal(back, x.astype(np.float64))
    assert np.array_equal(S.e4m3_decode(scales), sb)


def test_two_level_nvfp4_global_scale_from_the_tensor_max_keeps_block_scales_in_range():
    """With g = amax / (6 * 448) over the (rotated) tensor, no block scale
    saturates and the group holding the maximum uses the top of the UE4M3
    range, which is what the second level is for."""
    rng = np.random.default_rng(33)
    x = (rng.standard_normal((64, 256)) * 1e3).astype(np.float32)
    amax = np.float32(np.abs(Hd.fwht256_f32(x)).max())
    g = float(np.float32(amax / np.float32(6.0 * 448.0)))
    codes, scales = F.encode_rows("e2m1_g16", True, x, tensor_scale=g)
    sv = S.e4m3_decode(scales)
    assert sv.max() <= 448.0 and sv.max() >= 256.0
    # without the second level, these values saturate the block scales
    _, s1 = F.encode_rows("e2m1_g16", True, x, tensor_scale=1.0)
    assert S.e4m3_decode(s1).max() == 448.0


# ------------------------------------------------------------------ layout

@pytest.mark.parametrize("bits,D", [(16, 256), (16, 128), (8, 256), (8, 128), (4, 256)])
def test_code_layouts_are_bijections(bits, D):
    nbytes = 16 * D * bits // 8
    t = np.repeat(np.arange(16), D)
    d = np.tile(np.arange(D), 16)
    for pos_fn in (Lo.k_code_pos, Lo.v_code_pos):
        byte, hi = pos_fn(bits, t, d)
        per = 2 if bits == 16 else 1
        if bits == 4:
            key = byte * 2 + hi
            assert np.array_equal(np.sort(key), np.arange(2 * nbytes))
            owner = {}
            for b, tt, dd, h in zip(byte, t, d, hi):
                owner.setdefault(int(b), []).append((int(h), int(tt), int(dd)))
            for vals in owner.values():
                (h0, t0, d0), (h1, t1, d1) = sorted(vals)
                if pos_fn is Lo.k_code_pos:  # two consecutive values of one token
                    assert t0 == t1 and d1 == d0 + 1 and d0 % 2 == 0
                else:  # one column of an (even, odd) token pair, the even one low
                    assert d0 == d1 and t1 == t0 + 1 and t0 % 2 == 0
        else:
            assert np.array_equal(np.sort(byte), np.arange(0, nbytes, per))


def test_write_read_round_trip_and_isolation():
    rng = np.random.default_rng(25)
    for fmt in range(7):
        D = 128 if fmt == 5 else 256
        P = 128 if fmt == 5 else 64
        geo = Lo.Geometry(fmt, D, P, 2)
        pool = np.full(3 * geo.page_bytes, 0xA5, dtype=np.uint8)
        slots = rng.permutation(3 * P)[:37]
        kb = F.CODECS[geo.kc][0]
        vb = F.CODECS[geo.vc][0]
        mk = {16: 1 << 16, 8: 256, 4: 16}
        kc = rng.integers(0, mk[kb], (37, D))
        vc = rng.integers(0, mk[vb], (37, D))
        gk, gv = F.n_groups(geo.kc, D), F.n_groups(geo.vc, D)
        sk = {"f16": 1 << 16, "ue4m3": 256, "ue8m0": 256, None: 1}
        ks = None if gk == 0 else rng.integers(0, sk[F.CODECS[geo.kc][2]], (37, gk))
        vs = None if gv == 0 else rng.integers(0, sk[F.CODECS[geo.vc][2]], (37, gv))
        before = pool.copy()
        Lo.write_rows(pool, geo, slots, 1, kc, ks, vc, vs)
        rk, rks, rv, rvs = Lo.read_rows(pool, geo, slots, 1)
        assert np.array_equal(rk, kc) and np.array_equal(rv, vc)
        if ks is not None:
            assert np.array_equal(rks, ks)
        if vs is not None:
            assert np.array_equal(rvs, vs)
        # head 0 and every other slot untouched
        changed = np.flatnonzero(pool != before)
        mask = Lo.written_byte_mask(geo, 3, slots)
        assert np.all(mask[changed])
        other = np.setdiff1d(np.arange(3 * P), slots)
        r0 = Lo.read_rows(before, geo, other, 1)
        r1 = Lo.read_rows(pool, geo, other, 1)
        assert all(np.array_equal(a, b) for a, b in zip(r0, r1) if a is not None)


@pytest.mark.parametrize("fmt", [3, 4])
def test_token_pair_written_in_two_calls(fmt):
    """4-bit V bytes hold one column of two tokens: writing the two tokens of
    a pair in two calls, in either order, gives the bytes one call gives."""
    geo = Lo.Geometry(fmt, 256, 64, 2)
    rng = np.random.default_rng(31)
    slots = np.array([6, 7, 9, 8, 17, 40])  # pairs (6, 7), (8, 9); 17 and 40 alone
    kc = rng.integers(0, 256 if fmt == 4 else 16, (6, 256))
    vc = rng.integers(0, 16, (6, 256))
    ks = rng.integers(0, 1 << 16, (6, 1)) if fmt == 4 else rng.integers(0, 256, (6, 16))
    vs = rng.integers(0, 256, (6, 16))
    joint = np.full(geo.page_bytes, 0x3C, dtype=np.uint8)
    Lo.write_rows(joint, geo, slots, 1, kc, ks, vc, vs)
    for order in ([0, 2, 4, 5], [1, 3, 4, 5]), ([1, 3], [0, 2, 4, 5]):
        split = np.full(geo.page_bytes, 0x3C, dtype=np.uint8)
        for sel in order:
            Lo.write_rows(split, geo, slots[sel], 1, kc[sel], ks[sel], vc[sel], vs[sel])
        assert np.array_equal(split, joint)
