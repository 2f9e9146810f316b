"""GPU parity at the workloads' full sizes, in the launch configuration the
bench times (planned grid, split + combine), on sampled outputs.

The whole cache is written and read by the HIP path; for a few sampled
(sequence, kv head) units the oracle encodes that unit's K/V rows itself
(its own codecs, no layout), checks the bytes the GPU stored for them, and
computes the unit's attention outputs one by one.  Inputs are the seeded
workload generator's (drawn on the GPU, as in the bench); nothing the oracle
uses comes from the HIP path.
"""

import numpy as np
import pytest
import torch

import decode_attention_quant_amd as kvq
import workloads as W
from oracle import attention as OA, formats as OF, layout as OL
from oracle.scalar import bf16_bits_to_f32
from _gpu_common import assert_close, assert_lse_close, note, require_gpu

pytestmark = pytest.mark.gpu

# (workload config, format): every decode workload at its full size
CASES = [
    (2, "INT8_G64"),
    (2, "FP8_ROW"),
    (2, "FP8_TENSOR"),
    (3, "NVFP4_G16"),
    (3, "NVFP4_G16/2L"),  # calibrated per-tensor second-level scales
    (3, "MXFP4"),
    ("3b", "NVFP4_G16"),
    (4, "K8V4"),
    (5, "MXFP8"),
]


def sampled_units(c, n_rand=1, seed=17):
    lens = c.seq_lens
    units = {(int(np.argmax(lens)), 0), (int(np.argmin(lens)), c.H_kv - 1)}
    rng = np.random.default_rng(seed)
    while len(units) < 2 + n_rand:
        units.add((int(rng.integers(c.B)), int(rng.integers(c.H_kv))))
    return sorted(units)


def oracle_unit(c, geo, pool, b, h, q_mxfp8=False):
    """The oracle's encoding of unit (b, h) checked against the GPU bytes,
    then its attention outputs [n_q][G][D] and lse [n_q][G]."""
    start = int(c.seq_lens[:b].astype(np.int64).sum())
    L = int(c.seq_lens[b])
    G = c.H_q // c.H_kv
    kbits = W.bf16_bits(c.k[start:start + L, h])
    vbits = W.bf16_bits(c.v[start:start + L, h])
    kx = kbits if geo.kc == "bf16" else bf16_bits_to_f32(kbits)
    kc, ks = OF.encode_rows(geo.kc, geo.k_rot, kx, c.k_scale)
    vc, vs = OF.encode_rows(geo.vc, geo.v_rot, bf16_bits_to_f32(vbits), c.v_scale)
    # the GPU's bytes for these slots, read through the oracle's layout from
    # a copy of just this sequence's pages
    npg = -(-L // c.P)
    pages = c.block_table[b, :npg].astype(np.int64)
    mini = pool.view(c.num_pages, -1)[torch.as_tensor(pages, device=pool.device)].cpu().numpy().reshape(-1)
    pos = np.arange(L)
    got = OL.read_rows(mini, geo, (pos // c.P) * c.P + pos % c.P, h)
    for name, g, r in zip(("K codes", "K scales", "V codes", "V scales"), got, (kc, ks, vc, vs)):
        if r is None:
            continue
        assert np.array_equal(np.asarray(g).astype(np.int64), np.asarray(r).astype(np.int64)), \
            "unit (%d, %d): %s differ" % (b, h, name)
    K = OF.decode_rows(geo.kc, geo.k_rot, kc, ks, c.k_scale)
    V = OF.decode_rows(geo.vc, geo.v_rot, vc, vs, c.v_scale)
    q = bf16_bits_to_f32(W.bf16_bits(c.q[b, :, h * G:(h + 1) * G, :])).astype(np.float64)
    if q_mxfp8:
        q = OA.quantize_query_mxfp8(q)
    return OA.attend(q, K, V, c.softmax_scale, c.n_q)


def run_full(cfg, label, flags=0):
    require_gpu()
    note("full-size case", cfg, label)
    fmt, _, mod = label.partition("/")
    c = W.make_case(cfg, fmt, device="cuda", two_level=mod == "2L")
    geo = OL.Geometry(c.fmt, c.D, c.P, c.H_kv)
    d = kvq.desc(c.fmt, c.D, c.P, c.H_kv, c.num_pages, c.k_scale, c.v_scale)
    pool = kvq.alloc_pool(d)
    note("full-size append", cfg, fmt, "tokens", c.k.shape[0])
    kvq.quantize_append(d, pool, c.k, c.v, c.slot_mapping)
    bt = torch.as_tensor(c.block_table, device="cuda")
    sl = torch.as_tensor(c.seq_lens, device="cuda")
    ws = kvq.alloc_workspace(kvq.workspace_size(d, c.B, c.n_q, c.H_q, c.max_pages))
    out = torch.full((c.B, c.n_q, c.H_q, c.D), float("nan"), device="cuda")
    lse = torch.full((c.B, c.n_q, c.H_q), float("nan"), device="cuda")
    note("full-size decode (planned grid)", cfg, fmt, "nwg", kvq.decode_plan(d, c.B, c.n_q, c.H_q, c.max_pages)[0])
    fl = kvq.SPLIT_WRITE_WHOLE_UNITS | flags
    kvq.decode_split(d, pool, c.q, bt, sl, c.softmax_scale, ws, flags=fl, out=out, lse=lse)
    kvq.decode_combine(d, c.B, c.n_q, c.H_q, c.max_pages, sl, ws, out, lse, flags=fl)
    torch.cuda.synchronize()
    return c, geo, d, pool, bt, sl, ws, out, lse


@pytest.mark.parametrize("cfg,fmt", CASES)
def test_full_size_sampled_units(cfg, fmt):
    c, geo, d, pool, bt, sl, ws, out, lse = run_full(cfg, fmt)
    o_all, l_all = out.cpu().numpy(), lse.cpu().numpy()
    assert np.all(np.isfinite(o_all)) and np.all(np.isfinite(l_all)), "every row written"
    G = c.H_q // c.H_kv
    for b, h in sampled_units(c):
        note("oracle unit", cfg, fmt, (b, h), "length", int(c.seq_lens[b]))
        ref, ref_lse = oracle_unit(c, geo, pool, b, h)
        assert_close(o_all[b, :, h * G:(h + 1) * G, :], ref, "full-size %s %s unit (%d, %d)" % (cfg, fmt, b, h))
        assert_lse_close(l_all[b, :, h * G:(h + 1) * G], ref_lse, "full-size %s %s unit (%d, %d)" % (cfg, fmt, b, h))


@pytest.mark.parametrize("cfg,fmt", [(2, "INT8_G64"), (3, "NVFP4_G16"), (5, "MXFP8")])
def test_full_size_fused_step_equals_separate(cfg, fmt):
    """The bench's fused step (the newest n_q tokens of every sequence stored
    again, then decode, in the split launch) leaves the pool's bytes as they
    were and gives the separate path's outputs bit for bit."""
    c, geo, d, pool, bt, sl, ws, out, lse = run_full(cfg, fmt)
    lens = c.seq_lens.astype(np.int64)
    idx = torch.as_tensor(((np.cumsum(lens) - c.n_q)[:, None] + np.arange(c.n_q)[None, :]).reshape(-1),
                          device="cuda")
    k_new = c.k.index_select(0, idx).view(c.B, c.n_q, c.H_kv, c.D).contiguous()
    v_new = c.v.index_select(0, idx).view(c.B, c.n_q, c.H_kv, c.D).contiguous()
    before = pool.clone()
    out2 = torch.full_like(out, float("nan"))
    lse2 = torch.full_like(lse, float("nan"))
    note("full-size fused step", cfg, fmt)
    fl = kvq.SPLIT_WRITE_WHOLE_UNITS
    kvq.decode_step_split(d, pool, k_new, v_new, c.q, bt, sl, c.softmax_scale, ws, flags=fl, out=out2, lse=lse2)
    kvq.decode_combine(d, c.B, c.n_q, c.H_q, c.max_pages, sl, ws, out2, lse2, flags=fl)
    torch.cuda.synchronize()
    assert torch.equal(pool, before)
    assert torch.equal(out2.view(torch.int32), out.view(torch.int32))
    assert torch.equal(lse2.view(torch.int32), lse.view(torch.int32))


def test_full_size_query_mxfp8_mode():
    c, geo, d, pool, bt, sl, ws, out, lse = run_full(5, "MXFP8", flags=kvq.SPLIT_Q_MXFP8)
    o_all, l_all = out.cpu().numpy(), lse.cpu().numpy()
    G = c.H_q // c.H_kv
    for b, h in sampled_units(c):
        note("oracle unit (query-MXFP8 mode)", (b, h))
        ref, ref_lse = oracle_unit(c, geo, pool, b, h, q_mxfp8=True)
        assert_close(o_all[b, :, h * G:(h + 1) * G, :], ref, "full-size MTP query-MXFP8 unit (%d, %d)" % (b, h))
        assert_lse_close(l_all[b, :, h * G:(h + 1) * G], ref_lse, "full-size MTP query-MXFP8 unit (%d, %d)" % (b, h))


def test_full_size_chunk_append_and_prefill():
    """The bench's prefill workload at full size: 64 sequences of the mixed
    K8V4 cache each get a 2048-token chunk appended (the quant-append
    measurement), then the chunk's queries attend causally over the cache
    (the prefill measurement).  For sampled units the chunk's stored bytes
    are checked against the oracle's encoding, and sampled query rows
    against the oracle's attention."""
    require_gpu()
    chunk = 2048
    note("full-size prefill case")
    c = W.make_case(4, "K8V4", device="cuda", n_q=chunk, reserve=chunk)
    geo = OL.Geometry(c.fmt, c.D, c.P, c.H_kv)
    d = kvq.desc(c.fmt, c.D, c.P, c.H_kv, c.num_pages, c.k_scale, c.v_scale)
    pool = kvq.alloc_pool(d)
    kvq.quantize_append(d, pool, c.k, c.v, c.slot_mapping)
    k, v, slots = W.append_chunk(c, chunk, device="cuda")
    note("full-size chunk append", k.shape[0], "tokens")
    kvq.quantize_append(d, pool, k, v, slots)
    lens = c.seq_lens.astype(np.int64) + chunk
    bt = torch.as_tensor(c.block_table, device="cuda")
    sl = torch.as_tensor(lens.astype(np.int32), device="cuda")
    out = torch.full(c.q.shape, float("nan"), device="cuda")
    note("full-size prefill")
    kvq.prefill_attention(d, pool, c.q, bt, sl, c.softmax_scale, out=out)
    torch.cuda.synchronize()
    G = c.H_q // c.H_kv
    starts = np.concatenate([[0], np.cumsum(c.seq_lens.astype(np.int64))])
    for b, h in sampled_units(c):
        L0, L = int(c.seq_lens[b]), int(lens[b])
        note("oracle prefill unit", (b, h), "cached", L0)
        kb = np.concatenate([W.bf16_bits(c.k[starts[b]:starts[b + 1], h]), W.bf16_bits(k[b * chunk:(b + 1) * chunk, h])])
        vb = np.concatenate([W.bf16_bits(c.v[starts[b]:starts[b + 1], h]), W.bf16_bits(v[b * chunk:(b + 1) * chunk, h])])
        kc, ks = OF.encode_rows(geo.kc, geo.k_rot, bf16_bits_to_f32(kb), c.k_scale)
        vc, vs = OF.encode_rows(geo.vc, geo.v_rot, bf16_bits_to_f32(vb), c.v_scale)
        # the chunk's bytes as stored by the GPU
        npg = -(-L // c.P)
        pages = c.block_table[b, :npg].astype(np.int64)
        mini = pool.view(c.num_pages, -1)[torch.as_tensor(pages, device="cuda")].cpu().numpy().reshape(-1)
        new = np.arange(L0, L)
        got = OL.read_rows(mini, geo, new, h)
        for name, g, r in zip(("K codes", "K scales", "V codes", "V scales"), got, (kc, ks, vc, vs)):
            assert np.array_equal(np.asarray(g).astype(np.int64), np.asarray(r)[L0:].astype(np.int64)), \
                "chunk of unit (%d, %d): %s differ" % (b, h, name)
        K = OF.decode_rows(geo.kc, geo.k_rot, kc, ks, c.k_scale)
        V = OF.decode_rows(geo.vc, geo.v_rot, vc, vs, c.v_scale)
        q = bf16_bits_to_f32(W.bf16_bits(c.q[b, :, h * G:(h + 1) * G, :])).astype(np.float64)
        o = out[b, :, h * G:(h + 1) * G, :].cpu().numpy()
        for i in (0, chunk // 2 + 7, chunk - 1):  # query i sits at position L0 + i
            p = L0 + i
            ref, _ = OA.attend(q[i:i + 1], K[:p + 1], V[:p + 1], c.softmax_scale, 1)
            assert_close(o[i:i + 1], ref, "full-size prefill unit (%d, %d) query %d" % (b, h, i))
