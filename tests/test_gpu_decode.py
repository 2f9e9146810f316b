"""GPU parity of decode attention against the fp64 oracle.

Tolerance (north-star): |gpu - ref| <= 1e-3 + 2e-3 |ref| elementwise, with
the GPU accumulating in fp32.  Cases use every config's shapes at sizes the
oracle finishes in seconds, spanning several pages and a ragged tail, plus
edge lengths, split-count sweeps, determinism and page-permutation checks.
"""

import numpy as np
import pytest
import torch

import decode_attention_quant_amd as kvq
import workloads as W
from _gpu_common import (assert_close, assert_lse_close, build, note, oracle_attention, require_gpu, W_name)
import _schedule as S

pytestmark = pytest.mark.gpu

# (config, format, B, lengths)
CASES = [
    (1, "BF16", 1, [1024]),
    (1, "FP8_ROW", 1, [1024]),
    (2, "INT8_G64", 4, [1200, 700, 65, 333]),
    (2, "FP8_ROW", 4, [1200, 700, 65, 333]),
    (2, "FP8_TENSOR", 4, [1200, 700, 65, 333]),
    (3, "NVFP4_G16", 2, [2100, 900]),
    (4, "K8V4", 6, [1500, 20, 640, 129, 2000, 777]),
    (5, "MXFP8", 3, [700, 260, 128]),
    (3, "MXFP4", 2, [2100, 901]),
    (4, "MXFP4", 5, [1500, 21, 640, 129, 777]),
]


def run_decode(bl, lse=True):
    c = bl.case
    q = c.q.cuda()
    out = torch.full((c.B, c.n_q, c.H_q, c.D), float("nan"), dtype=torch.float32, device="cuda")
    l = torch.full((c.B, c.n_q, c.H_q), float("nan"), dtype=torch.float32, device="cuda") if lse else None
    note("decode", W_name(c))
    kvq.decode_attention(bl.desc, bl.pool_gpu, q, bl.bt, bl.sl, c.softmax_scale, out=out, lse=l)
    torch.cuda.synchronize()
    return out.cpu().numpy(), (l.cpu().numpy() if lse else None)


@pytest.mark.parametrize("cfg,fmt,B,lens", CASES)
def test_decode_matches_oracle(cfg, fmt, B, lens):
    c = W.make_case(cfg, fmt, device="cpu", B=B, lengths=lens)
    bl = build(c)
    out, lse = run_decode(bl)
    ref, ref_lse = oracle_attention(bl)
    assert_close(out, ref, W_name(c))
    assert_lse_close(lse, ref_lse, W_name(c))


# Query-row shapes beyond the workloads': R = G * n_q rows share a kv head.
# R = 1 is MHA with one query token; R = 24 is the 24 / 4 GQA group with 4
# MTP tokens and R = 40 a 40 / 4 group with 4, which take two and three
# 16-row tiles (the second and third tiles, blockIdx.y > 0, the last one
# partly filled).  (config, format, n_q, H_q, H_kv)
ROW_SHAPES = [
    (1, "BF16", 1, 2, 2), (2, "INT8_G64", 1, 4, 4), (2, "FP8_ROW", 1, 4, 4), (2, "FP8_TENSOR", 1, 4, 4),
    (3, "NVFP4_G16", 1, 4, 4), (4, "K8V4", 1, 4, 4), (5, "MXFP8", 1, None, None), (3, "MXFP4", 1, 4, 4),
    (1, "BF16", 4, 24, 4), (2, "INT8_G64", 4, None, None), (2, "FP8_ROW", 4, None, None),
    (2, "FP8_TENSOR", 4, None, None), (3, "NVFP4_G16", 4, None, None), (4, "K8V4", 4, None, None),
    (5, "MXFP8", 4, 192, 32), (3, "MXFP4", 4, None, None), (4, "K8V4", 4, 40, 4), (2, "INT8_G64", 4, 40, 4),
]


@pytest.mark.parametrize("cfg,fmt,n_q,H_q,H_kv", ROW_SHAPES)
def test_query_row_shapes(cfg, fmt, n_q, H_q, H_kv):
    lens = [700, 130, 3] if cfg != 5 else [700, 258, 3]
    c = W.make_case(cfg, fmt, device="cpu", B=3, lengths=lens, n_q=n_q, H_q=H_q, H_kv=H_kv)
    assert (c.H_q // c.H_kv) * c.n_q in (1, 24, 40)
    bl = build(c)
    out, lse = run_decode(bl)
    ref, ref_lse = oracle_attention(bl)
    assert_close(out, ref, W_name(c))
    assert_lse_close(lse, ref_lse, W_name(c))
    # the split path with forced workgroup counts merges every tile's partials
    q = c.q.cuda()
    for nwg in (5, 64):
        ws = kvq.alloc_workspace(kvq.workspace_size(bl.desc, c.B, c.n_q, c.H_q, c.max_pages, nwg))
        ws.fill_(0xFF)
        o2 = torch.full((c.B, c.n_q, c.H_q, c.D), float("nan"), device="cuda")
        l2 = torch.full((c.B, c.n_q, c.H_q), float("nan"), device="cuda")
        note("row shapes split", W_name(c), "nwg", nwg)
        kvq.decode_split(bl.desc, bl.pool_gpu, q, bl.bt, bl.sl, c.softmax_scale, ws, num_workgroups=nwg,
                         flags=kvq.SPLIT_WRITE_WHOLE_UNITS, out=o2, lse=l2)
        kvq.decode_combine(bl.desc, c.B, c.n_q, c.H_q, c.max_pages, bl.sl, ws, o2, l2, num_workgroups=nwg,
                           flags=kvq.SPLIT_WRITE_WHOLE_UNITS)
        torch.cuda.synchronize()
        assert_close(o2.cpu().numpy(), ref, "%s nwg=%d" % (W_name(c), nwg))
        assert_lse_close(l2.cpu().numpy(), ref_lse, "%s nwg=%d" % (W_name(c), nwg))


@pytest.mark.parametrize("fmt,cfg", [("INT8_G64", 2), ("FP8_ROW", 2), ("MXFP8", 5), ("MXFP4", 3), ("BF16", 1),
                                     ("NVFP4_G16", 3), ("K8V4", 4)])
def test_values_at_the_edge_of_the_supported_range(fmt, cfg):
    """V up to just below 2^15 in magnitude (the supported range of the
    formats whose V is expanded to fp16 with its scale, include/kvq.h):
    every decoded value stays inside fp16 and the outputs match the oracle.
    V is the recipe's N(0, 1) draw times S = 12000, so outputs are compared
    after dividing by S: the tolerance's absolute term is set for unit-scale
    values, and the relative errors of the path do not depend on the scale."""
    c = W.make_case(cfg, fmt, device="cpu", B=2, lengths=[700, 130])
    v = (c.v.float() * 12000.0).clamp(-32512.0, 32512.0)
    v[::97, :, ::17] = 32512.0   # the largest bf16 below 2^15, spread over tokens and dims
    v[5::97, :, 3::19] = -32512.0
    c.v = v.to(torch.bfloat16)
    assert float(c.v.float().abs().max()) < 32768.0
    bl = build(c)
    out, lse = run_decode(bl)
    ref, ref_lse = oracle_attention(bl)
    assert np.all(np.isfinite(out))
    assert_close(out / 12000.0, ref / 12000.0, "large V " + W_name(c))
    assert_lse_close(lse, ref_lse, "large V " + W_name(c))


def test_fp8_tensor_unit_scale():
    c = W.make_case(2, "FP8_TENSOR", device="cpu", B=2, lengths=[300, 90], calibrate_tensor_scale=False)
    assert c.k_scale == 1.0 and c.v_scale == 1.0
    bl = build(c)
    out, lse = run_decode(bl)
    ref, ref_lse = oracle_attention(bl)
    assert_close(out, ref, "fp8 tensor unit scale")


@pytest.mark.parametrize("fmt,cfg", [("FP8_ROW", 2), ("NVFP4_G16", 3), ("MXFP8", 5), ("K8V4", 4), ("INT8_G64", 2),
                                     ("MXFP4", 3)])
def test_edge_lengths(fmt, cfg):
    lens = [0, 1, 15, 16, 17, 63, 64, 65, 127, 128, 129, 3]
    c = W.make_case(cfg, fmt, device="cpu", B=len(lens), lengths=lens)
    bl = build(c)
    out, lse = run_decode(bl)
    ref, ref_lse = oracle_attention(bl)
    assert_close(out, ref, W_name(c))
    assert_lse_close(lse, ref_lse, W_name(c))
    assert np.all(out[0] == 0) and np.all(np.isneginf(lse[0]))


def test_mtp_short_sequences():
    """n_q = 4 with sequences shorter than 4: early queries see nothing."""
    lens = [2, 4, 5, 300]
    c = W.make_case(5, "MXFP8", device="cpu", B=4, lengths=lens)
    bl = build(c)
    out, lse = run_decode(bl)
    ref, ref_lse = oracle_attention(bl)
    assert_close(out, ref, "mtp short")
    assert_lse_close(lse, ref_lse, "mtp short")
    assert np.all(out[0, :2] == 0)


@pytest.mark.parametrize("fmt,cfg", [("INT8_G64", 2), ("NVFP4_G16", 3), ("MXFP8", 5), ("K8V4", 4),
                                     ("MXFP4", 3)])
def test_workgroup_sweep_and_phases(fmt, cfg):
    """Any number of split workgroups (ranges that cut units anywhere, one
    workgroup holding many units, empty workgroups) gives the same answer,
    through the two-phase API as through the one-call one."""
    c = W.make_case(cfg, fmt, device="cpu", B=3, lengths=[900, 450, 77] if cfg != 5 else [1100, 450, 77])
    bl = build(c)
    ref, ref_lse = oracle_attention(bl)
    q = c.q.cuda()
    for nwg in (1, 2, 3, 7, 64, 333, 0):
        for flags in (0, kvq.SPLIT_WRITE_WHOLE_UNITS):
            ws = kvq.alloc_workspace(kvq.workspace_size(bl.desc, c.B, c.n_q, c.H_q, c.max_pages, nwg))
            ws.fill_(0xFF)  # workspace contents on entry must not matter
            out = torch.full((c.B, c.n_q, c.H_q, c.D), float("nan"), device="cuda")
            lse = torch.full((c.B, c.n_q, c.H_q), float("nan"), device="cuda")
            note("workgroup sweep", fmt, "nwg", nwg, "flags", flags)
            kvq.decode_split(bl.desc, bl.pool_gpu, q, bl.bt, bl.sl, c.softmax_scale, ws, num_workgroups=nwg,
                             flags=flags, out=out, lse=lse)
            kvq.decode_combine(bl.desc, c.B, c.n_q, c.H_q, c.max_pages, bl.sl, ws, out, lse, num_workgroups=nwg,
                               flags=flags)
            torch.cuda.synchronize()
            assert_close(out.cpu().numpy(), ref, "%s nwg=%d flags=%d" % (fmt, nwg, flags))
            assert_lse_close(lse.cpu().numpy(), ref_lse, "%s nwg=%d flags=%d" % (fmt, nwg, flags))


def merge_documented_partials(ws, c, nwg, seg_cost=S.SEG_COST):
    """Merge the split phase's partials as kvq.h documents them: the schedule
    (units' blocks with seg_cost positions between units, exact shares over
    the workgroups that get work), slot u + w per (unit, workgroup), and the
    (m, l, o) layout of the workspace."""
    B, H, D = c.B, c.H_kv, c.D
    G = c.H_q // H
    R = G * c.n_q
    units = B * H
    slots = units + nwg
    a256 = lambda n: (n + 255) // 256 * 256
    raw = ws.cpu().numpy()
    cum = raw[: 4 * (B + 1)].view(np.int32)
    o_ml = a256(4 * (B + 1))
    ml = raw[o_ml: o_ml + 8 * slots * R].view(np.float32).reshape(slots, R, 2)
    o_o = o_ml + a256(8 * slots * R)
    o = raw[o_o: o_o + 4 * slots * R * D].view(np.float32).reshape(slots, R, D)
    T = int(cum[B])
    C = T + seg_cost * max(units - 1, 0)
    n = S.ways(C, nwg)
    owner = lambda y: S.owner(C, n, y)
    out = np.zeros((B, c.n_q, c.H_q, D))
    lse = np.full((B, c.n_q, c.H_q), -np.inf)
    for b in range(B):
        nb = (int(c.seq_lens[b]) + 15) // 16
        assert cum[b] == H * sum((int(L) + 15) // 16 for L in c.seq_lens[:b])
        for h in range(H):
            if nb == 0:
                continue
            u = b * H + h
            start = int(cum[b]) + h * nb + seg_cost * u
            ws_ = range(owner(start), owner(start + nb - 1) + 1)
            for r in range(R):
                m = np.array([ml[u + w, r, 0] for w in ws_], np.float64)
                l = np.array([ml[u + w, r, 1] for w in ws_], np.float64)
                ov = np.array([o[u + w, r] for w in ws_], np.float64)
                M = m.max()
                f = np.where(np.isneginf(m), 0.0, np.exp2(m - M))
                L = (f * l).sum()
                i, j = divmod(r, G)
                out[b, i, h * G + j] = (f[:, None] * ov).sum(0) / L
                lse[b, i, h * G + j] = (M + np.log2(L)) * np.log(2.0)
    return out, lse


@pytest.mark.parametrize("fmt,cfg,lens", [("K8V4", 4, [900, 450, 77, 0, 1]), ("MXFP8", 5, [1100, 450, 77])])
def test_partials_follow_the_documented_schedule(fmt, cfg, lens):
    """The partials a caller may merge itself sit where the header says:
    merged here by that description alone (numpy), they give the oracle's
    attention, for forced and planned workgroup counts.  (Formats without a
    per-tensor V scale, which the combine applies when it normalizes.)"""
    c = W.make_case(cfg, fmt, device="cpu", B=len(lens), lengths=lens)
    bl = build(c)
    ref, ref_lse = oracle_attention(bl)
    q = c.q.cuda()
    planned, _ = kvq.decode_plan(bl.desc, c.B, c.n_q, c.H_q, c.max_pages)
    for nwg in (1, 5, 37, 333, 0):
        ws = kvq.alloc_workspace(kvq.workspace_size(bl.desc, c.B, c.n_q, c.H_q, c.max_pages, nwg))
        ws.fill_(0xFF)
        note("documented partials", fmt, "nwg", nwg)
        kvq.decode_split(bl.desc, bl.pool_gpu, q, bl.bt, bl.sl, c.softmax_scale, ws, num_workgroups=nwg, flags=0)
        torch.cuda.synchronize()
        out, lse = merge_documented_partials(ws, c, nwg or planned)
        live = np.asarray(c.seq_lens) > 0
        assert_close(out[live], ref[live], "%s nwg=%d" % (fmt, nwg))
        assert_lse_close(lse[live], ref_lse[live], "%s nwg=%d" % (fmt, nwg))


@pytest.mark.parametrize("fmt,cfg", [("K8V4", 4), ("FP8_ROW", 2)])
def test_deterministic_and_permutation_invariant(fmt, cfg):
    lens = [700, 300, 65]
    c = W.make_case(cfg, fmt, device="cpu", B=3, lengths=lens, extra_pages=5)
    bl = build(c, oracle=False)
    a, la = run_decode(bl)
    b, lb = run_decode(bl)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32)) and np.array_equal(la.view(np.uint32),
                                                                                  lb.view(np.uint32))
    # same data under another physical page assignment: identical results
    perm = np.random.default_rng(5).permutation(c.num_pages).astype(np.int32)
    c2 = W.make_case(cfg, fmt, device="cpu", B=3, lengths=lens, extra_pages=5)
    c2.block_table = perm[c2.block_table]
    seq, pos = c2.token_seq, c2.token_pos
    c2.slot_mapping = torch.as_tensor((c2.block_table[seq, pos // c2.P].astype(np.int64) * c2.P + pos % c2.P)
                                      .astype(np.int32))
    bl2 = build(c2, oracle=False)
    d, ld = run_decode(bl2)
    assert np.array_equal(a.view(np.uint32), d.view(np.uint32))


@pytest.mark.parametrize("fill", [0x7F, 0xFF, 0x00])
def test_slack_slots_hold_garbage(fill):
    """Unwritten slots past the end (here NaN code patterns) never leak in."""
    c = W.make_case(4, "K8V4", device="cpu", B=3, lengths=[70, 33, 129])
    bl = build(c, fill=fill)
    out, lse = run_decode(bl)
    ref, ref_lse = oracle_attention(bl)
    assert np.all(np.isfinite(out))
    assert_close(out, ref, "fill %#x" % fill)


@pytest.mark.parametrize("nwg", [300, 64])
def test_many_partials_per_unit_head_dim_128(nwg):
    """head_dim 128 (MXFP8, 32 kv heads) with one sequence split over many
    workgroups: the combine merges tens of partials per unit side by side."""
    c = W.make_case(5, "MXFP8", device="cpu", B=1, lengths=[3000])
    bl = build(c)
    ref, ref_lse = oracle_attention(bl)
    q = c.q.cuda()
    ws = kvq.alloc_workspace(kvq.workspace_size(bl.desc, c.B, c.n_q, c.H_q, c.max_pages, nwg))
    ws.fill_(0xFF)
    out = torch.full((c.B, c.n_q, c.H_q, c.D), float("nan"), device="cuda")
    lse = torch.full((c.B, c.n_q, c.H_q), float("nan"), device="cuda")
    note("combine d128", "nwg", nwg)
    kvq.decode_split(bl.desc, bl.pool_gpu, q, bl.bt, bl.sl, c.softmax_scale, ws, num_workgroups=nwg,
                     flags=kvq.SPLIT_WRITE_WHOLE_UNITS, out=out, lse=lse)
    kvq.decode_combine(bl.desc, c.B, c.n_q, c.H_q, c.max_pages, bl.sl, ws, out, lse, num_workgroups=nwg,
                       flags=kvq.SPLIT_WRITE_WHOLE_UNITS)
    torch.cuda.synchronize()
    assert_close(out.cpu().numpy(), ref, "mxfp8 nwg=%d" % nwg)
    assert_lse_close(lse.cpu().numpy(), ref_lse, "mxfp8 nwg=%d" % nwg)


def test_combine_over_a_hundred_partials():
    """One 60000-token sequence over 2 kv heads split 1024 ways: about 125
    partials per unit, so the combine's threads each hold 8 partials in
    flight (and the rest take the tail path)."""
    c = W.make_case(1, "FP8_ROW", device="cpu", B=1, lengths=[60000])
    bl = build(c)
    ref, ref_lse = oracle_attention(bl)
    q = c.q.cuda()
    nwg = 1024
    ws = kvq.alloc_workspace(kvq.workspace_size(bl.desc, c.B, c.n_q, c.H_q, c.max_pages, nwg))
    ws.fill_(0xFF)
    out = torch.full((c.B, c.n_q, c.H_q, c.D), float("nan"), device="cuda")
    lse = torch.full((c.B, c.n_q, c.H_q), float("nan"), device="cuda")
    note("combine many partials", "nwg", nwg)
    kvq.decode_split(bl.desc, bl.pool_gpu, q, bl.bt, bl.sl, c.softmax_scale, ws, num_workgroups=nwg,
                     flags=kvq.SPLIT_WRITE_WHOLE_UNITS, out=out, lse=lse)
    kvq.decode_combine(bl.desc, c.B, c.n_q, c.H_q, c.max_pages, bl.sl, ws, out, lse, num_workgroups=nwg,
                       flags=kvq.SPLIT_WRITE_WHOLE_UNITS)
    torch.cuda.synchronize()
    assert_close(out.cpu().numpy(), ref, "many partials")
    assert_lse_close(lse.cpu().numpy(), ref_lse, "many partials")


@pytest.mark.parametrize("fmt,cfg", [("NVFP4_G16", 3), ("FP8_ROW", 2), ("INT8_G64", 2), ("K8V4", 4), ("MXFP8", 5),
                                     ("BF16", 1), ("MXFP4", 3)])
def test_scores_that_climb_and_jump(fmt, cfg):
    """Keys scaled up along each sequence (up to 6x at the end) with a few
    6x spikes late on: the running maximum climbs block after block and
    jumps by far more than the rescale slack mid-stream, so the kernel both
    runs with probabilities above 1 and rescales l and O part-way."""
    c = W.make_case(cfg, fmt, device="cpu", B=2, lengths=[1500, 700])
    pos = torch.as_tensor(c.token_pos, dtype=torch.float32)
    L = torch.as_tensor(c.seq_lens[c.token_seq].astype(np.float32))
    factor = 1.0 + 5.0 * pos / L
    late = np.flatnonzero(c.token_pos > 0.6 * c.seq_lens[c.token_seq])
    factor[np.random.default_rng(11).choice(late, size=6, replace=False)] *= 6.0
    c.k = (c.k.float() * factor[:, None, None]).to(torch.bfloat16)
    bl = build(c)
    out, lse = run_decode(bl)
    ref, ref_lse = oracle_attention(bl)
    assert_close(out, ref, "climbing scores " + W_name(c))
    assert_lse_close(lse, ref_lse, "climbing scores " + W_name(c))


def test_planned_grid_is_one_round():
    """The planner's grid: one round of resident workgroups (a multiple of
    the CU count), whatever the cache's size and its number of units."""
    require_gpu()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    one, _ = kvq.decode_plan(kvq.desc(3, 256, 64, 4, 4097), 1, 1, 24, 4096)        # 4 units x 16384 blocks
    big, _ = kvq.decode_plan(kvq.desc(3, 256, 64, 4, 16385), 32, 1, 24, 512)       # 128 units x 2048 blocks
    many, slots = kvq.decode_plan(kvq.desc(5, 128, 128, 32, 8193), 256, 4, 32, 32)  # 8192 units x 256 blocks
    assert one % cus == 0 and one // cus >= 1
    assert big == one and many == one and slots == 256 * 32 + one
