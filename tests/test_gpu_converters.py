"""GPU parity of the element conversions the encoders rest on, swept past
the workloads' values and compared byte for byte with the oracle.

The encoders turn each quotient x / scale into a code with the hardware's
packed conversions (fp32 -> E4M3 for the FP8 formats, fp32 -> E2M1 for the
4-bit ones, fp32 -> fp16 for BF16's V), so the bit-exact codec bar (the
NInfer guide's FP8-E4M3 and NVFP4-G16 entries; TokenSpeed's fp8_e4m3 with a
per-tensor scale) holds only if those conversions round to nearest even and
saturate exactly as the formats' definitions say, at every grid midpoint
and one float32 step on either side.  Every call goes through
kvq_quantize_append; the expected bytes are the oracle's.

  * BF16: every finite bf16 value as K (kept bitwise) and V (IEEE fp16,
    overflow to infinity, fp16 subnormals);
  * FP8_TENSOR: every finite bf16 value under 256 per-tensor scales from
    2^-40 to 2^40 (powers of two and not; the encoder's fast division covers
    [2^-30, 2^30] and IEEE division the rest), saturation included;
  * FP8_TENSOR, targeted: per-tensor scales searched so that x / scale is
    exactly each E4M3 grid value and each midpoint between neighbours (and
    the 464 saturation boundary), its float32 predecessor and successor, both
    signs;
  * NVFP4_G16, two-level NVFP4, MXFP4 and K8V4's V (all Hadamard-rotated
    before quantization): rows (c0, c0, c2, c3, 0, ...) rotate, in the fixed
    fp32 butterfly order, into groups that hold +-(c2 - c3) / 16 exactly next
    to an element that pins the group scale to a power of two, so the E2M1
    conversion sees exactly each E2M1 grid value and midpoint, their float32
    neighbours and the saturation range; the construction is checked with
    the oracle's own rotation before any GPU work.
"""

import numpy as np
import pytest
import torch

import decode_attention_quant_amd as kvq
import workloads as W
from oracle import attention as OA, formats as OF, hadamard as OH, layout as OL, scalar as OS
from _gpu_common import note, require_gpu

pytestmark = pytest.mark.gpu

D = 256


def finite_bf16():
    """Every finite bf16 bit pattern (65,280 of them), as [255][256] rows."""
    bits = np.arange(1 << 16, dtype=np.uint32)
    keep = ((bits >> 7) & 0xFF) != 0xFF
    return bits[keep].astype(np.uint16).reshape(-1, D)


def bf16_of(x):
    """bf16 bits of float32 values that bf16 holds exactly."""
    b = np.asarray(x, dtype=np.float32).reshape(-1).view(np.uint32)
    assert np.all((b & 0xFFFF) == 0), "not a bf16 value"
    return (b >> 16).astype(np.uint16).reshape(np.shape(x))


def run_calls(fmt, calls, P=64):
    """calls: (k_bits [T][1][D] uint16, v_bits, k_scale, v_scale, first slot).
    All calls go to one pool of one kv head; returns (gpu bytes, oracle bytes)."""
    require_gpu()
    fid = W.FORMAT_IDS[fmt]
    end = max(s0 + k.shape[0] for k, _, _, _, s0 in calls)
    num_pages = -(-end // P)
    geo = OL.Geometry(fid, D, P, 1)
    pool = torch.full((num_pages * geo.page_bytes,), 0xA5, dtype=torch.uint8, device="cuda")
    ref = np.full(num_pages * geo.page_bytes, 0xA5, dtype=np.uint8)
    note("converter sweep", fmt, "calls", len(calls), "pages", num_pages)
    for k, v, ks, vs, s0 in calls:
        d = kvq.desc(fmt, D, P, 1, num_pages, ks, vs)
        slots = np.arange(s0, s0 + k.shape[0], dtype=np.int32)
        kt = torch.from_numpy(k.view(np.int16).copy()).view(torch.bfloat16).cuda()
        vt = torch.from_numpy(v.view(np.int16).copy()).view(torch.bfloat16).cuda()
        kvq.quantize_append(d, pool, kt, vt, torch.from_numpy(slots).cuda())
        with np.errstate(over="ignore", invalid="ignore", divide="ignore"):
            OA.quantize_append(geo, ref, k, v, slots, ks, vs)
    torch.cuda.synchronize()
    return pool.cpu().numpy(), ref


def assert_same(got, ref, what):
    diff = np.flatnonzero(got != ref)
    assert diff.size == 0, "%s: %d bytes differ, first at %s: got %s ref %s" % (
        what, diff.size, diff[:8], got[diff[:8]], ref[diff[:8]])


def test_bf16_every_value():
    rows = finite_bf16()[:, None, :]
    got, ref = run_calls("BF16", [(rows, rows[::-1].copy(), 1.0, 1.0, 0)])
    assert_same(got, ref, "BF16: every finite bf16 value")


def tensor_scales():
    """256 per-tensor scales: every power of two 2^-30 .. 2^30, four outside
    the fast division's range, the range's inner neighbours, and log-uniform
    non-powers of two in [2^-30, 2^30]."""
    s = [2.0 ** e for e in range(-30, 31)]
    s += [2.0 ** -40, 2.0 ** -31, 2.0 ** 31, 2.0 ** 40]
    s += [float(np.nextafter(np.float32(2.0 ** 30), np.float32(0))),
          float(np.nextafter(np.float32(2.0 ** -30), np.float32(1)))]
    rng = np.random.default_rng(2024)
    while len(s) < 256:
        x = np.float32(2.0 ** rng.uniform(-30, 30))
        if x != np.float32(2.0) ** np.round(np.log2(x)):
            s.append(float(x))
    return s


def test_fp8_tensor_every_value_under_256_scales():
    rows = finite_bf16()[:, None, :]
    perm = np.random.default_rng(7).permutation(rows.size)
    vrows = rows.reshape(-1)[perm].reshape(rows.shape)
    sc = tensor_scales()
    assert len(sc) == 256 and len(set(sc)) == 256
    calls = []
    for i in range(0, 256, 2):
        calls.append((rows, vrows, sc[i], sc[i + 1], (i // 2) * 256))
    got, ref = run_calls("FP8_TENSOR", calls)
    assert_same(got, ref, "FP8_TENSOR: every finite bf16 value under 256 scales")


def e4m3_targets():
    """Every positive E4M3 grid value, every midpoint between neighbours and
    the 464 saturation boundary, each with its float32 neighbours."""
    grid = np.unique(np.abs(OS.e4m3_decode(np.arange(0x7F)))).astype(np.float64)  # 0 .. 448
    mids = (grid[:-1] + grid[1:]) / 2
    pts = np.concatenate([grid[1:], mids, [464.0]]).astype(np.float32)
    t = np.concatenate([pts, np.nextafter(pts, np.float32(0)), np.nextafter(pts, np.float32(np.inf))])
    return np.unique(t)


def scale_for(t, x_candidates):
    """(x, s): bf16 x and fp32 s with fl(x / s) == t (IEEE float32 division),
    searched over the scales within 8 float32 steps of x / t."""
    t = np.float32(t)
    for x in x_candidates:
        x = np.float32(x)
        s0 = np.float32(x / t)
        lo = hi = s0
        cand = [s0]
        for _ in range(8):
            lo = np.nextafter(lo, np.float32(0))
            hi = np.nextafter(hi, np.float32(np.inf))
            cand += [lo, hi]
        for s in cand:
            if np.float32(x / s) == t:
                return x, s
    raise AssertionError("no scale found for %r" % t)


def numerators(base):
    """bf16 values base * m, m running over the 128 bf16 mantissas in [1, 2)."""
    return [np.float32(base * (1.0 + k / 128.0)) for k in range(128)]


def test_fp8_tensor_e4m3_midpoints_and_neighbours():
    """The quotient x / scale lands exactly on each target, both signs; the
    other 255 elements of the row are random finite bf16 values at that
    scale.  About one target in eight takes a scale outside [2^-30, 2^30],
    where the encoder divides with the IEEE sequence."""
    targets = e4m3_targets()
    rng = np.random.default_rng(99)
    bf = finite_bf16().reshape(-1)
    xs_fast = numerators(1.0)
    xs_slow = numerators(2.0 ** 40)
    picks = []
    for i, t in enumerate(targets):
        for sign in (1.0, -1.0):
            cands = xs_slow if i % 8 == 0 else xs_fast
            x, s = scale_for(t, cands)
            assert np.float32(np.float32(sign * x) / s) == np.float32(sign * t)
            picks.append((np.float32(sign * x), s))
    calls = []
    for j in range(0, len(picks) - 1, 2):
        rows = []
        for x, _ in picks[j:j + 2]:
            r = rng.choice(bf, size=D)
            r[0] = bf16_of(x)
            rows.append(r.reshape(1, 1, D))
        calls.append((rows[0], rows[1], float(picks[j][1]), float(picks[j + 1][1]), j // 2))
    got, ref = run_calls("FP8_TENSOR", calls)
    assert_same(got, ref, "FP8_TENSOR: %d E4M3 targets" % len(picks))


# ---- 4-bit formats: the quotient the E2M1 conversion sees, set exactly

E2M1_POINTS = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def e2m1_targets(limit):
    """(p, t): bf16 values p and quotients t, t = p or one of p's float32
    neighbours: the E2M1 grid values and midpoints, the saturation range up
    to `limit` (the largest quotient the group scale rule leaves) and a few
    values in between and near zero."""
    out = []
    for p in E2M1_POINTS:
        p = np.float32(p)
        out += [(p, np.nextafter(p, np.float32(0))), (p, p), (p, np.nextafter(p, np.float32(np.inf)))]
    extra = [6.125, 6.25, 6.375, 7.0, 7.5, 7.875, 0.0, 2.0 ** -20, 0.125, 0.2490234375, 0.75390625, 2.75,
             4.5, 5.5]
    out += [(np.float32(v), np.float32(v)) for v in extra]
    return [(p, t) for p, t in out if t <= limit]


def row_for(p, t):
    """Row (c0, c0, c2, c3, 0, ...) of bf16 values, c2 = p and c3 = p - t (a
    power of two or zero), so that c2 - c3 == t exactly in float32, and
    2 c0 + c2 + c3 close to 6 (c0 = 0 past 6).  Its rotation holds
    +-(c2 - c3) / 16 in every group next to 2 c0 +- (c2 + c3) over 16."""
    c2 = np.float32(p)
    c3 = np.float32(c2 - np.float32(t))
    assert np.float32(c2 - c3) == np.float32(t)
    c0 = np.float32(max(6.0 - float(t), 0.0) / 2)
    c0 = (c0.view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32)  # a bf16 value, rounded toward zero
    r = np.zeros(D, np.float32)
    r[:4] = [c0, c0, c2, c3]
    bf16_of(r)  # every element is a bf16 value
    return r


def check_rotated_plane(rows, mx, g, want, sign):
    """The oracle's rotation and group scales of `rows`: a power-of-two scale
    s in every group and the quotients +-t at positions 1 and 3."""
    y = OH.fwht256_f32(rows)
    _, sb = OF.encode_rows("e2m1_mx32" if mx else "e2m1_g16", True, rows, tensor_scale=g)
    scale = (OS.ue8m0_decode(sb) if mx else OS.e4m3_decode(sb)).astype(np.float64)
    for i in range(rows.shape[0]):
        s0 = scale[i, 0]
        assert s0 > 0 and np.log2(s0) == np.round(np.log2(s0)) and np.all(scale[i] == s0), (i, scale[i])
        q1 = np.float32(np.float32(y[i, 1] / np.float32(g)) / np.float32(s0))
        q3 = np.float32(np.float32(y[i, 3] / np.float32(g)) / np.float32(s0))
        assert q1 == sign * want[i] and q3 == -sign * want[i], (i, want[i], q1, q3)


# (format, per-tensor scales of the K and V planes, row multipliers 2^j
# that keep every group scale a power of two inside its format's range)
E2M1_CASES = [
    ("NVFP4_G16", 1.0, 1.0, (0, -5, 12)),
    ("NVFP4_G16", 2.0 ** -3, 2.0 ** 5, (0, 3, 9)),  # two-level NVFP4
    ("MXFP4", 1.0, 1.0, (0, -24, 12)),
    ("K8V4", 1.0, 1.0, (0, -5, 12)),               # V only (K is FP8 row-256)
]


@pytest.mark.parametrize("fmt,ks,vs,js", E2M1_CASES)
def test_e2m1_midpoints_and_neighbours(fmt, ks, vs, js):
    mx = fmt == "MXFP4"
    targets = e2m1_targets(7.9 if mx else 6.375)
    rows, want = [], []
    for p, t in targets:
        base = row_for(p, t)
        for j in js:
            rows.append((base * np.float32(2.0 ** j)).astype(np.float32))
            want.append(np.float32(t))
    rows = np.stack(rows)
    if fmt != "K8V4":
        check_rotated_plane(rows, mx, ks, want, 1.0)
    check_rotated_plane(-rows, mx, vs, want, -1.0)
    kb = bf16_of(rows)[:, None, :]
    vb = bf16_of(-rows)[:, None, :]
    got, ref = run_calls(fmt, [(kb, vb, ks, vs, 0)])
    assert_same(got, ref, "%s (scales %g, %g): %d E2M1 targets x %d group scales" % (
        fmt, ks, vs, len(targets), len(js)))
