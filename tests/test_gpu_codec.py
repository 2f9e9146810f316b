"""GPU parity: quantize-append writes exactly the oracle's bytes, and
dequant-page returns exactly the oracle's stored values (bit for bit)."""

import numpy as np
import pytest
import torch

import decode_attention_quant_amd as kvq
import workloads as W
from oracle import attention as OA, layout as OL, formats as OF
from _gpu_common import build, note, require_gpu, W_name

pytestmark = pytest.mark.gpu

# (format, config whose shapes it borrows, head_dim override)
CASES = [
    ("BF16", 1, None), ("FP8_ROW", 1, None), ("INT8_G64", 2, None), ("FP8_ROW", 2, None), ("FP8_TENSOR", 2, None),
    ("NVFP4_G16", 3, None), ("K8V4", 4, None), ("MXFP8", 5, None), ("MXFP4", 3, None), ("MXFP4", 4, None),
]


# quantize_append takes its single-token kernel (a wave per token and kv
# head) for calls of at most this many tokens and its 16-token row kernel
# above; the tests below run on both sides of it.
TOKEN_KERNEL_MAX_T = 256
KERNELS = ["token", "rows"]


def _mismatch(bl):
    got = bl.pool_gpu.cpu().numpy()
    ref = bl.pool_ref
    diff = np.flatnonzero(got != ref)
    return got, ref, diff


@pytest.mark.parametrize("kernel", KERNELS)
@pytest.mark.parametrize("fmt,cfg,_", CASES)
def test_append_bytes_bit_exact(fmt, cfg, _, kernel):
    lens = [130, 65, 7, 1] if kernel == "token" else [330, 65, 7, 1]
    assert (sum(lens) <= TOKEN_KERNEL_MAX_T) == (kernel == "token")
    c = W.make_case(cfg, fmt, device="cpu", B=4, lengths=lens)
    bl = build(c)
    got, ref, diff = _mismatch(bl)
    assert diff.size == 0, "%s: %d bytes differ, first at %s: got %s ref %s" % (
        W_name(c), diff.size, diff[:8], got[diff[:8]], ref[diff[:8]])
    # bytes of slots that were never written keep the pool's fill
    mask = OL.written_byte_mask(bl.geo, c.num_pages, c.slot_mapping.numpy())
    assert np.all(got[~mask] == 0xFF)


@pytest.mark.parametrize("fmt", ["BF16", "FP8_ROW", "FP8_TENSOR", "MXFP8"])
def test_append_head_dim_128(fmt):
    # config 5's shapes: head_dim 128, 128-token pages, 32 kv heads
    c = W.make_case(5, fmt, device="cpu", B=3, lengths=[200, 129, 3])
    bl = build(c)
    got, ref, diff = _mismatch(bl)
    assert diff.size == 0, "%s: %d bytes differ" % (W_name(c), diff.size)


def _adversarial_rows(D, rng):
    """Rows built to hit ties, saturation, zeros, signed zeros and subnormals."""
    rows = []
    f32 = np.float32
    # E4M3 grid midpoints scaled so that amax/448 is a power of two (exact scale)
    grid = np.unique(np.abs(OF.S.e4m3_decode(np.arange(127))))
    mids = (grid[:-1] + grid[1:]) / 2
    r = np.zeros(D, f32)
    r[: min(D, len(mids))] = mids[:D]
    r[-1] = 448.0
    rows.append(r)
    rows.append(-r)
    # E2M1 ties inside 16-groups whose amax is 6 (scale 1)
    t = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, 0.0, -0.0, -0.25, -2.5, -5.0, 0.5, 1.0, 6.0], f32)
    rows.append(np.tile(t, D // 16))
    # int8 ties: amax 127 with x.5 values
    r = (np.arange(D) % 127 - 63).astype(f32) + 0.5
    r[0] = 127.0
    rows.append(r)
    rows.append(np.zeros(D, f32))                         # all zero
    r = np.zeros(D, f32)
    r[5] = -0.0
    r[7] = 1e-30
    rows.append(r)                                        # tiny amax
    rows.append((rng.standard_normal(D) * 1e-38).astype(f32))   # fp32 subnormal range
    r = rng.standard_normal(D).astype(f32)
    r[3] = 3.0e4
    rows.append(r)                                        # huge outlier
    rows.append((rng.standard_normal(D) * 6e4).astype(f32))     # near the fp16 limit
    rows.append(np.full(D, 1.0, f32))                     # constant
    return np.stack(rows)


@pytest.mark.parametrize("kernel", KERNELS)
@pytest.mark.parametrize("fmt", ["INT8_G64", "FP8_ROW", "NVFP4_G16", "K8V4", "MXFP8", "FP8_TENSOR", "BF16", "MXFP4"])
def test_append_adversarial_rows_bit_exact(fmt, kernel):
    require_gpu()
    D, P, H = 256, 64, 2
    rng = np.random.default_rng(77)
    rows = _adversarial_rows(D, rng)
    if kernel == "rows":  # the rows again, scaled by powers of two, past the single-token limit
        rows = np.concatenate([rows * np.float32(2.0 ** (i % 5 - 2)) for i in range(27)])
    n = rows.shape[0]
    assert (n <= TOKEN_KERNEL_MAX_T) == (kernel == "token")
    x = np.stack([rows, rows[::-1] * np.float32(0.5)], axis=1)  # [n][H][D]
    xt = torch.from_numpy(x).to(torch.bfloat16)
    k_scale = v_scale = 0.37
    pages = -(-n // P)
    d = kvq.desc(fmt, D, P, H, pages, k_scale, v_scale)
    geo = OL.Geometry(W.FORMAT_IDS[fmt], D, P, H)
    slots = torch.arange(n, dtype=torch.int32)
    pool = kvq.alloc_pool(d)
    note("append adversarial", fmt, kernel)
    kvq.quantize_append(d, pool, xt.cuda(), xt.flip(0).contiguous().cuda(), slots.cuda())
    torch.cuda.synchronize()
    ref = np.full(pages * geo.page_bytes, 0xFF, np.uint8)
    OA.quantize_append(geo, ref, W.bf16_bits(xt), W.bf16_bits(xt.flip(0)), slots.numpy(), k_scale, v_scale)
    got = pool.cpu().numpy()
    diff = np.flatnonzero(got != ref)
    assert diff.size == 0, "%s: %d bytes differ at %s: got %s ref %s" % (fmt, diff.size, diff[:8], got[diff[:8]],
                                                                        ref[diff[:8]])


def test_negative_slots_are_skipped():
    c = W.make_case(2, "FP8_ROW", device="cpu", B=2, lengths=[70, 20])
    c.slot_mapping[::3] = -1
    bl = build(c)
    got, ref, diff = _mismatch(bl)
    assert diff.size == 0


@pytest.mark.parametrize("fmt,cfg", [(f, c) for f, c, _ in CASES])
def test_dequant_page_bit_exact_stored_domain(fmt, cfg):
    c = W.make_case(cfg, fmt, device="cpu", B=2, lengths=[c_len(cfg), 17])
    bl = build(c)
    for page in range(c.num_pages):
        note("dequant", fmt, "page", page)
        k, v = kvq.dequant_page(bl.desc, bl.pool_gpu, page, stored_domain=True)
        K, V = OA.dequant_page(bl.geo, bl.pool_ref, page, c.k_scale, c.v_scale, stored_domain=True)
        kg, vg = k.cpu().numpy(), v.cpu().numpy()
        # compare only written slots (others hold canary bytes, possibly NaN codes)
        slots = set(c.slot_mapping.numpy().tolist())
        rows = [s - page * c.P for s in range(page * c.P, (page + 1) * c.P) if s in slots]
        for K_, kg_ in ((K, kg), (V, vg)):
            a = K_[:, rows].astype(np.float32)
            b = kg_[:, rows]
            assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), "%s page %d" % (fmt, page)


def c_len(cfg):
    return 200 if cfg != 5 else 300


@pytest.mark.parametrize("fmt,cfg", [("INT8_G64", 2), ("NVFP4_G16", 3), ("K8V4", 4), ("MXFP4", 3)])
def test_dequant_page_original_domain(fmt, cfg):
    c = W.make_case(cfg, fmt, device="cpu", B=1, lengths=[128])
    bl = build(c)
    for page in range(c.num_pages):
        k, v = kvq.dequant_page(bl.desc, bl.pool_gpu, page, stored_domain=False)
        K, V = OA.dequant_page(bl.geo, bl.pool_ref, page, stored_domain=False)
        assert np.allclose(k.cpu().numpy(), K, atol=1e-5 * np.abs(K).max(), rtol=1e-5)
        assert np.allclose(v.cpu().numpy(), V, atol=1e-5 * np.abs(V).max(), rtol=1e-5)


@pytest.mark.parametrize("fmt,cfg", [("K8V4", 4), ("NVFP4_G16", 3), ("INT8_G64", 2), ("FP8_ROW", 2),
                                     ("FP8_TENSOR", 2), ("BF16", 1), ("MXFP8", 5), ("MXFP4", 3)])
@pytest.mark.parametrize("chunk", [37, 75])
def test_append_chunks_at_any_offset(fmt, cfg, chunk):
    """Prefill chunks appended after cached prefixes start at every alignment
    inside a 16-slot block and a 4-slot slab (consecutive slots, shifted),
    the layout of the bench's prefill workload; the pool stays bit-exact.
    4 chunks of 37 tokens take the single-token kernel, of 75 the rows."""
    lens = [5, 70, 130, 3] if cfg != 5 else [5, 134, 66, 3]
    c = W.make_case(cfg, fmt, device="cpu", B=4, lengths=lens, reserve=chunk)
    bl = build(c)
    k, v, slots = W.append_chunk(c, chunk)
    note("append chunk", W_name(c), "chunk", chunk)
    kvq.quantize_append(bl.desc, bl.pool_gpu, k.cuda(), v.cuda(), slots.cuda())
    torch.cuda.synchronize()
    OA.quantize_append(bl.geo, bl.pool_ref, W.bf16_bits(k), W.bf16_bits(v), slots.numpy(), c.k_scale, c.v_scale)
    got, ref, diff = _mismatch(bl)
    assert diff.size == 0, "%s: %d bytes differ, first at %s: got %s ref %s" % (
        W_name(c), diff.size, diff[:8], got[diff[:8]], ref[diff[:8]])
    # the chunks really start at every slab alignment
    starts = slots.numpy()[np.arange(4) * chunk]
    assert sorted(set((starts % 4).tolist())) == [1, 2, 3] or len(set((starts % 4).tolist())) >= 2


@pytest.mark.parametrize("fmt,cfg", [("NVFP4_G16", 3), ("K8V4", 4), ("INT8_G64", 2), ("FP8_ROW", 2), ("MXFP8", 5),
                                     ("BF16", 1), ("MXFP4", 4)])
@pytest.mark.parametrize("kernel", KERNELS)
def test_append_slots_in_random_order(fmt, cfg, kernel):
    """One call writes every slot of a few pages in random input order, so the
    tokens that share a slab (and, for 4-bit V, a byte) sit in different rows
    and waves and are stored concurrently, token by token."""
    require_gpu()
    c = W.make_case(cfg, fmt, device="cpu", B=1, lengths=[8])
    geo = OL.Geometry(c.fmt, c.D, c.P, c.H_kv)
    num_pages = TOKEN_KERNEL_MAX_T // c.P + (kernel == "rows")
    d = kvq.desc(c.fmt, c.D, c.P, c.H_kv, num_pages, c.k_scale, c.v_scale)
    n = num_pages * c.P
    gen = torch.Generator().manual_seed(41)
    k = (torch.randn((n, c.H_kv, c.D), generator=gen) * 2.0).to(torch.bfloat16)
    v = torch.randn((n, c.H_kv, c.D), generator=gen).to(torch.bfloat16)
    slots = torch.as_tensor(np.random.default_rng(41).permutation(n).astype(np.int32))
    pool = kvq.alloc_pool(d, fill=0x5A)
    note("append random order", fmt, kernel)
    kvq.quantize_append(d, pool, k.cuda(), v.cuda(), slots.cuda())
    torch.cuda.synchronize()
    ref = np.full(num_pages * geo.page_bytes, 0x5A, np.uint8)
    OA.quantize_append(geo, ref, W.bf16_bits(k), W.bf16_bits(v), slots.numpy(), c.k_scale, c.v_scale)
    got = pool.cpu().numpy()
    diff = np.flatnonzero(got != ref)
    assert diff.size == 0, "%s: %d bytes differ at %s: got %s ref %s" % (fmt, diff.size, diff[:8], got[diff[:8]],
                                                                        ref[diff[:8]])


@pytest.mark.parametrize("fmt,cfg", [("NVFP4_G16", 3), ("K8V4", 4), ("FP8_ROW", 2), ("MXFP4", 3)])
def test_single_token_steps_and_rewrites(fmt, cfg):
    """Decode-style appends of one token per sequence, step after step (the
    even and odd tokens of each 4-bit V byte pair arrive in different calls),
    and a rewrite of an already written slot with new values after each step
    (a rejected draft token): the pool matches the oracle after every call."""
    lens = [6, 65, 11]
    steps = 5
    c = W.make_case(cfg, fmt, device="cpu", B=3, lengths=lens, reserve=steps)
    bl = build(c)
    k_all, v_all, slots_all = W.append_chunk(c, steps)
    slots_all = slots_all.numpy().reshape(c.B, steps)
    k_all = k_all.reshape(c.B, steps, c.H_kv, c.D)
    v_all = v_all.reshape(c.B, steps, c.H_kv, c.D)
    gen = torch.Generator().manual_seed(43)
    for s in range(steps):
        k, v = k_all[:, s].contiguous(), v_all[:, s].contiguous()
        sl = torch.as_tensor(slots_all[:, s].copy())
        calls = [(k, v, sl)]
        # rewrite the token just written to sequence s % B with other values
        b = s % c.B
        calls.append(((torch.randn((1, c.H_kv, c.D), generator=gen) * 3.0).to(torch.bfloat16),
                      torch.randn((1, c.H_kv, c.D), generator=gen).to(torch.bfloat16),
                      torch.as_tensor(slots_all[b:b + 1, s].copy())))
        for kk, vv, ss in calls:
            note("single token step", fmt, "step", s, "slots", ss.tolist())
            kvq.quantize_append(bl.desc, bl.pool_gpu, kk.cuda(), vv.cuda(), ss.cuda())
            torch.cuda.synchronize()
            OA.quantize_append(bl.geo, bl.pool_ref, W.bf16_bits(kk), W.bf16_bits(vv), ss.numpy(), c.k_scale,
                               c.v_scale)
            got, ref, diff = _mismatch(bl)
            assert diff.size == 0, "%s step %d: %d bytes differ at %s: got %s ref %s" % (
                fmt, s, diff.size, diff[:8], got[diff[:8]], ref[diff[:8]])
