"""GPU parity of two-level NVFP4: NVFP4 planes with a per-tensor fp32 scale
above their 16-value UE4M3 scales (the descriptor's k_scale / v_scale for
NVFP4_G16, v_scale for K8V4's V).  The write path must give the oracle's
bytes, and every read path (split decode, fused step, prefill, page
dequantization) the oracle's values."""

import numpy as np
import pytest
import torch

import decode_attention_quant_amd as kvq
import workloads as W
from oracle import attention as OA
from _gpu_common import assert_close, assert_lse_close, build, note, oracle_attention, W_name

pytestmark = pytest.mark.gpu

# (config, format, k_scale, v_scale): a power of two, tensor-max calibrated
# values, and a scale far from 1
SCALES = [
    (3, "NVFP4_G16", 2.0 ** -5, 2.0 ** -3),
    (3, "NVFP4_G16", 0.03711, 0.02137),
    (4, "K8V4", 1.0, 0.0179),
    (4, "K8V4", 1.0, 7.5),
]


def two_level_case(cfg, fmt, ks, vs, lens, **kw):
    c = W.make_case(cfg, fmt, device="cpu", B=len(lens), lengths=lens, **kw)
    c.k_scale, c.v_scale = ks, vs
    return c


@pytest.mark.parametrize("cfg,fmt,ks,vs", SCALES)
def test_two_level_append_bit_exact_and_decode(cfg, fmt, ks, vs):
    c = two_level_case(cfg, fmt, ks, vs, [301, 77, 16])
    bl = build(c)
    got = bl.pool_gpu.cpu().numpy()
    diff = np.flatnonzero(got != bl.pool_ref)
    assert diff.size == 0, "%s: %d bytes differ, first %s" % (W_name(c), diff.size, diff[:8])
    q = c.q.cuda()
    out = torch.full(q.shape, float("nan"), device="cuda")
    lse = torch.full(q.shape[:3], float("nan"), device="cuda")
    note("two-level decode", W_name(c), ks, vs)
    kvq.decode_attention(bl.desc, bl.pool_gpu, q, bl.bt, bl.sl, c.softmax_scale, out=out, lse=lse)
    torch.cuda.synchronize()
    ref, ref_lse = oracle_attention(bl)
    assert_close(out.cpu().numpy(), ref, "two-level " + W_name(c))
    assert_lse_close(lse.cpu().numpy(), ref_lse, "two-level " + W_name(c))


@pytest.mark.parametrize("cfg,fmt,ks,vs", SCALES[1:3])
def test_two_level_scale_changes_the_bytes(cfg, fmt, ks, vs):
    """The second level is really applied: the same rows at scale 1 encode
    to different bytes (and the oracle agrees with both)."""
    c = two_level_case(cfg, fmt, ks, vs, [200])
    bl = build(c)
    c1 = two_level_case(cfg, fmt, 1.0, 1.0, [200])
    bl1 = build(c1)
    assert np.array_equal(bl.pool_gpu.cpu().numpy(), bl.pool_ref)
    assert np.array_equal(bl1.pool_gpu.cpu().numpy(), bl1.pool_ref)
    assert not np.array_equal(bl.pool_ref, bl1.pool_ref)


@pytest.mark.parametrize("cfg,fmt,ks,vs", [SCALES[1], SCALES[2]])
def test_two_level_fused_step_and_prefill(cfg, fmt, ks, vs):
    n_new = W.CONFIGS[cfg]["n_q"]
    c = two_level_case(cfg, fmt, ks, vs, [640, 95], reserve=n_new)
    bl = build(c)
    k, v, slots = W.append_chunk(c, n_new)
    sl_new = torch.as_tensor(c.seq_lens + n_new, dtype=torch.int32, device="cuda")
    q = c.q.cuda()
    B, n_q, H_q, D = q.shape
    pool = bl.pool_gpu.clone()
    out = torch.full(q.shape, float("nan"), device="cuda")
    note("two-level fused step", W_name(c))
    kvq.decode_step(bl.desc, pool, k.view(B, n_q, c.H_kv, D).cuda(), v.view(B, n_q, c.H_kv, D).cuda(), q, bl.bt,
                    sl_new, c.softmax_scale, out=out)
    torch.cuda.synchronize()
    ref_pool = bl.pool_ref.copy()
    OA.quantize_append(bl.geo, ref_pool, W.bf16_bits(k), W.bf16_bits(v), slots.numpy(), ks, vs)
    assert np.array_equal(pool.cpu().numpy(), ref_pool)
    ref, _ = OA.attention_ref(bl.geo, ref_pool, W.bf16_bits(c.q), c.block_table, sl_new.cpu().numpy(),
                              c.softmax_scale, c.n_q, ks, vs)
    assert_close(out.cpu().numpy(), ref, "two-level fused step " + W_name(c))
    # prefill: a 21-token chunk over the same cache
    chunk = 21
    c2 = two_level_case(cfg, fmt, ks, vs, [300, 40], n_q=chunk, reserve=chunk)
    bl2 = build(c2)
    k2, v2, s2 = W.append_chunk(c2, chunk)
    kvq.quantize_append(bl2.desc, bl2.pool_gpu, k2.cuda(), v2.cuda(), s2.cuda())
    OA.quantize_append(bl2.geo, bl2.pool_ref, W.bf16_bits(k2), W.bf16_bits(v2), s2.numpy(), ks, vs)
    sl2 = (c2.seq_lens + chunk).astype(np.int32)
    out2 = torch.full(c2.q.shape, float("nan"), device="cuda")
    note("two-level prefill", W_name(c2))
    kvq.prefill_attention(bl2.desc, bl2.pool_gpu, c2.q.cuda(), bl2.bt, torch.as_tensor(sl2, device="cuda"),
                          c2.softmax_scale, out=out2)
    torch.cuda.synchronize()
    ref2, _ = OA.attention_ref(bl2.geo, bl2.pool_ref, W.bf16_bits(c2.q), c2.block_table, sl2, c2.softmax_scale,
                               c2.n_q, ks, vs)
    assert_close(out2.cpu().numpy(), ref2, "two-level prefill " + W_name(c2))


@pytest.mark.parametrize("cfg,fmt,ks,vs", [SCALES[1], SCALES[3]])
def test_two_level_dequant_page(cfg, fmt, ks, vs):
    c = two_level_case(cfg, fmt, ks, vs, [128])
    bl = build(c)
    for page in range(c.num_pages):
        for stored in (True, False):
            note("two-level dequant", fmt, page, stored)
            k, v = kvq.dequant_page(bl.desc, bl.pool_gpu, page, stored_domain=stored)
            K, V = OA.dequant_page(bl.geo, bl.pool_ref, page, ks, vs, stored_domain=stored)
            if stored:
                assert np.array_equal(K.astype(np.float32).view(np.uint32), k.cpu().numpy().view(np.uint32))
                assert np.array_equal(V.astype(np.float32).view(np.uint32), v.cpu().numpy().view(np.uint32))
            else:
                assert np.allclose(k.cpu().numpy(), K, atol=1e-5 * np.abs(K).max(), rtol=1e-5)
                assert np.allclose(v.cpu().numpy(), V, atol=1e-5 * np.abs(V).max(), rtol=1e-5)
