"""GPU parity of the fused decode step (append the n_q newest tokens and
attend, in one split launch plus the reduce).

The same step runs twice from one cache: through kvq_quantize_append +
kvq_decode_attention, and through kvq_decode_step.  The pools must agree
byte for byte and the outputs bit for bit, and both must match the oracle
(the oracle's append of the new tokens, then fp64 attention) within the
decode tolerance.
"""

import numpy as np
import pytest
import torch

import decode_attention_quant_amd as kvq
import workloads as W
from oracle import attention as OA
from _gpu_common import assert_close, assert_lse_close, build, note, W_name

pytestmark = pytest.mark.gpu


def step_both_ways(c, bl, n_new):
    """Run one step both ways; returns (out, lse, pool) of each and the new seq_lens."""
    k, v, slots = W.append_chunk(c, n_new)
    sl_new = torch.as_tensor(c.seq_lens + n_new, dtype=torch.int32, device="cuda")
    q = c.q.cuda()
    B, n_q, H_q, D = q.shape
    assert n_q == n_new
    res = []
    for fused in (False, True):
        pool = bl.pool_gpu.clone()
        out = torch.full((B, n_q, H_q, D), float("nan"), device="cuda")
        lse = torch.full((B, n_q, H_q), float("nan"), device="cuda")
        note("decode step", "fused" if fused else "separate", W_name(c))
        if fused:
            kvq.decode_step(bl.desc, pool, k.view(B, n_q, c.H_kv, D).cuda(), v.view(B, n_q, c.H_kv, D).cuda(), q,
                            bl.bt, sl_new, c.softmax_scale, out=out, lse=lse)
        else:
            kvq.quantize_append(bl.desc, pool, k.cuda(), v.cuda(), slots.cuda())
            kvq.decode_attention(bl.desc, pool, q, bl.bt, sl_new, c.softmax_scale, out=out, lse=lse)
        torch.cuda.synchronize()
        res.append((out.cpu().numpy(), lse.cpu().numpy(), pool.cpu().numpy()))
    return res, (k, v, slots), sl_new.cpu().numpy()


def check_step(c, bl, n_new):
    (sep, fus), (k, v, slots), sl_new = step_both_ways(c, bl, n_new)
    diff = np.flatnonzero(sep[2] != fus[2])
    assert diff.size == 0, "%s: pools differ in %d bytes, first at %s" % (W_name(c), diff.size, diff[:8])
    assert np.array_equal(sep[0].view(np.uint32), fus[0].view(np.uint32)), "outputs differ " + W_name(c)
    assert np.array_equal(sep[1].view(np.uint32), fus[1].view(np.uint32)), "lse differ " + W_name(c)
    # the oracle: its own append of the new tokens, then attention
    ref_pool = bl.pool_ref.copy()
    OA.quantize_append(bl.geo, ref_pool, W.bf16_bits(k), W.bf16_bits(v), slots.numpy(), c.k_scale, c.v_scale)
    diff = np.flatnonzero(ref_pool != fus[2])
    assert diff.size == 0, "%s: pool differs from the oracle's in %d bytes" % (W_name(c), diff.size)
    ref, ref_lse = OA.attention_ref(bl.geo, ref_pool, W.bf16_bits(c.q), c.block_table, sl_new, c.softmax_scale,
                                    c.n_q, c.k_scale, c.v_scale)
    assert_close(fus[0], ref, "fused step " + W_name(c))
    assert_lse_close(fus[1], ref_lse, "fused step " + W_name(c))
    return sl_new


# (config, format, cached lengths before the step)
CASES = [
    (1, "BF16", [1023]),
    (1, "FP8_ROW", [1000]),
    (2, "INT8_G64", [1199, 700, 64, 14]),       # new tokens at block offsets 15, 12, 0, 14
    (2, "FP8_ROW", [1199, 700, 64, 14]),
    (2, "FP8_TENSOR", [1199, 700, 64, 14]),
    (3, "NVFP4_G16", [2099, 900, 15]),           # odd positions: 4-bit V byte pairs half filled
    (4, "K8V4", [1500, 19, 640, 128, 2001, 776]),
    (5, "MXFP8", [700, 258, 124, 2]),            # n_q = 4: the 4 new tokens cross a block at 124 + 4
    (3, "MXFP4", [2099, 900, 15]),
]


@pytest.mark.parametrize("cfg,fmt,lens", CASES)
def test_fused_step_equals_append_then_decode(cfg, fmt, lens):
    n_new = W.CONFIGS[cfg]["n_q"]
    c = W.make_case(cfg, fmt, device="cpu", B=len(lens), lengths=lens, reserve=n_new)
    bl = build(c)
    check_step(c, bl, n_new)


@pytest.mark.parametrize("cfg,fmt,H_q,H_kv", [(2, "FP8_ROW", 4, 4), (3, "NVFP4_G16", 4, 4), (4, "K8V4", 4, 4),
                                           (5, "MXFP8", None, None), (2, "INT8_G64", 4, 4)])
def test_fused_step_single_query_row(cfg, fmt, H_q, H_kv):
    """G * n_q = 1 (MHA, one query token per step): one live row in the tile."""
    c = W.make_case(cfg, fmt, device="cpu", B=3, lengths=[700, 129, 14], n_q=1, H_q=H_q, H_kv=H_kv, reserve=1)
    assert (c.H_q // c.H_kv) * c.n_q == 1
    bl = build(c)
    check_step(c, bl, 1)


@pytest.mark.parametrize("cfg,fmt,n_q,H_q,H_kv", [(3, "NVFP4_G16", 4, 4, 4), (4, "K8V4", 3, 4, 4),
                                                  (2, "INT8_G64", 5, 2, 2), (5, "MXFP8", 8, None, None),
                                                  (1, "BF16", 6, 2, 2)])
def test_fused_step_many_new_tokens(cfg, fmt, n_q, H_q, H_kv):
    """More new tokens per sequence than the kernel loads ahead (2 rows at
    head_dim 256, 4 at 128): the rest are loaded and encoded one by one, and
    the new tokens of a sequence may span two blocks (two owner waves)."""
    c = W.make_case(cfg, fmt, device="cpu", B=3, lengths=[701, 126, 9], n_q=n_q, H_q=H_q, H_kv=H_kv, reserve=n_q)
    assert (c.H_q // c.H_kv) * c.n_q <= 16
    bl = build(c)
    check_step(c, bl, n_q)


def test_fused_step_rejects_more_than_one_row_tile():
    """G * n_q = 24 (24 / 4 GQA with 4 MTP tokens) takes two row tiles, so a
    block has two reading workgroups and the fused step is refused (the
    separate append + decode serve it); nothing is stored."""
    c = W.make_case(2, "FP8_ROW", device="cpu", B=2, lengths=[300, 40], n_q=4, reserve=4)
    bl = build(c, oracle=False)
    k, v, _ = W.append_chunk(c, 4)
    sl = torch.as_tensor(c.seq_lens + 4, dtype=torch.int32, device="cuda")
    pool = bl.pool_gpu.clone()
    note("fused step, two row tiles: refused")
    with pytest.raises(kvq.KvqError) as e:
        kvq.decode_step(bl.desc, pool, k.view(2, 4, c.H_kv, c.D).cuda(), v.view(2, 4, c.H_kv, c.D).cuda(),
                        c.q.cuda(), bl.bt, sl, c.softmax_scale)
    assert e.value.status == 2
    torch.cuda.synchronize()
    assert torch.equal(pool, bl.pool_gpu)


def test_fused_step_short_and_empty_sequences():
    """MTP with sequences shorter than n_q (new tokens at negative positions are
    not stored and see nothing) and one with no tokens at all."""
    c = W.make_case(5, "MXFP8", device="cpu", B=3, lengths=[0, 0, 300], reserve=4)
    bl = build(c)
    (sep, fus), _, _ = step_both_ways(c, bl, 4)
    assert np.array_equal(sep[2], fus[2])
    assert np.array_equal(sep[0].view(np.uint32), fus[0].view(np.uint32))
    # seq_lens 4, 4, 304 after the step: every new token is stored and visible
    c2 = W.make_case(5, "MXFP8", device="cpu", B=2, lengths=[0, 9], reserve=4)
    bl2 = build(c2)
    k, v, slots = W.append_chunk(c2, 4)
    sl = torch.as_tensor([2, 13], dtype=torch.int32, device="cuda")  # sequence 0: only 2 of its 4 new tokens
    q = c2.q.cuda()
    outs = []
    for fused in (False, True):
        pool = bl2.pool_gpu.clone()
        out = torch.full(q.shape, float("nan"), device="cuda")
        note("short step", fused)
        if fused:
            kvq.decode_step(bl2.desc, pool, k.view(2, 4, c2.H_kv, c2.D).cuda(), v.view(2, 4, c2.H_kv, c2.D).cuda(),
                            q, bl2.bt, sl, c2.softmax_scale, out=out)
        else:
            # positions seq_lens - 4 + i < 0 are skipped: sequence 0 stores its tokens 2, 3 at positions 0, 1
            s = slots.numpy().copy().reshape(2, 4)
            pos0 = np.arange(4) - 2
            s[0] = np.where(pos0 >= 0, c2.block_table[0, 0] * c2.P + np.maximum(pos0, 0), -1)
            s[1] = c2.block_table[1, 0] * c2.P + 9 + np.arange(4)
            kvq.quantize_append(bl2.desc, pool, k.cuda(), v.cuda(), torch.as_tensor(s.reshape(-1)).cuda())
            kvq.decode_attention(bl2.desc, pool, q, bl2.bt, sl, c2.softmax_scale, out=out)
        torch.cuda.synchronize()
        outs.append((out.cpu().numpy(), pool.cpu().numpy()))
    assert np.array_equal(outs[0][1], outs[1][1])
    assert np.array_equal(outs[0][0].view(np.uint32), outs[1][0].view(np.uint32))
    assert np.all(outs[1][0][0, :2] == 0)  # queries before position 0 see nothing


@pytest.mark.parametrize("fmt,cfg", [("NVFP4_G16", 3), ("K8V4", 4), ("INT8_G64", 2), ("MXFP4", 3)])
def test_fused_steps_in_a_row(fmt, cfg):
    """Three steps in a row, each appending one token per sequence, so the
    4-bit V byte pairs are completed by a later launch."""
    c = W.make_case(cfg, fmt, device="cpu", B=3, lengths=[31, 64, 5], reserve=3)
    bl = build(c)
    for s in range(3):
        check_step(c, bl, 1)
        # the step's result becomes the cache on both sides
        k, v, slots = W.append_chunk(c, 1)
        note("advance", s)
        kvq.quantize_append(bl.desc, bl.pool_gpu, k.cuda(), v.cuda(), slots.cuda())
        OA.quantize_append(bl.geo, bl.pool_ref, W.bf16_bits(k), W.bf16_bits(v), slots.numpy(), c.k_scale,
                           c.v_scale)
        c.seq_lens = c.seq_lens + 1
        c.reserve -= 1


@pytest.mark.parametrize("fmt,cfg", [("NVFP4_G16", 3), ("MXFP8", 5), ("K8V4", 4), ("FP8_ROW", 2), ("INT8_G64", 2),
                                     ("MXFP4", 3)])
@pytest.mark.parametrize("nwg", [1, 3])
def test_fused_step_with_long_ranges(fmt, cfg, nwg):
    """Few split workgroups, so each wave walks tens of blocks and its block
    holding the new tokens comes late in its ring (copied without a wait of
    its own after the stores): pools byte-identical and outputs bit-identical
    to append then decode with the same split."""
    n_new = W.CONFIGS[cfg]["n_q"]
    lens = [3001, 1500, 62] if cfg != 5 else [3001, 1500, 124, 2]
    c = W.make_case(cfg, fmt, device="cpu", B=len(lens), lengths=lens, reserve=n_new)
    bl = build(c, oracle=False)
    k, v, slots = W.append_chunk(c, n_new)
    sl_new = torch.as_tensor(c.seq_lens + n_new, dtype=torch.int32, device="cuda")
    q = c.q.cuda()
    B, n_q, H_q, D = q.shape
    res = []
    for fused in (False, True):
        pool = bl.pool_gpu.clone()
        ws = kvq.alloc_workspace(kvq.workspace_size(bl.desc, B, n_q, H_q, c.max_pages, nwg))
        out = torch.full((B, n_q, H_q, D), float("nan"), device="cuda")
        lse = torch.full((B, n_q, H_q), float("nan"), device="cuda")
        note("long-range step", fmt, "nwg", nwg, "fused" if fused else "separate")
        if fused:
            kvq.decode_step_split(bl.desc, pool, k.view(B, n_q, c.H_kv, D).cuda(), v.view(B, n_q, c.H_kv, D).cuda(),
                                  q, bl.bt, sl_new, c.softmax_scale, ws, num_workgroups=nwg,
                                  flags=kvq.SPLIT_WRITE_WHOLE_UNITS, out=out, lse=lse)
        else:
            kvq.quantize_append(bl.desc, pool, k.cuda(), v.cuda(), slots.cuda())
            kvq.decode_split(bl.desc, pool, q, bl.bt, sl_new, c.softmax_scale, ws, num_workgroups=nwg,
                             flags=kvq.SPLIT_WRITE_WHOLE_UNITS, out=out, lse=lse)
        kvq.decode_combine(bl.desc, B, n_q, H_q, c.max_pages, sl_new, ws, out, lse, num_workgroups=nwg,
                           flags=kvq.SPLIT_WRITE_WHOLE_UNITS)
        torch.cuda.synchronize()
        res.append((out.cpu().numpy(), lse.cpu().numpy(), pool.cpu().numpy()))
    (o0, l0, p0), (o1, l1, p1) = res
    diff = np.flatnonzero(p0 != p1)
    assert diff.size == 0, "%s: pools differ in %d bytes" % (fmt, diff.size)
    assert np.array_equal(o0.view(np.uint32), o1.view(np.uint32)), "outputs differ " + fmt
    assert np.array_equal(l0.view(np.uint32), l1.view(np.uint32)), "lse differ " + fmt
