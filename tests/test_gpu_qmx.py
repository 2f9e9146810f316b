"""GPU parity of the query-MXFP8 mode of MXFP8 caches: the split phase with
KVQ_SPLIT_Q_MXFP8 rounds each query row to MXFP8 and runs Q.K on the
block-scaled fp8 MFMA; the result must be the oracle's attention of the
rounded query (``attention_ref(..., q_mxfp8=True)``)."""

import numpy as np
import pytest
import torch

import decode_attention_quant_amd as kvq
import workloads as W
from oracle import attention as OA
from _gpu_common import ATOL, RTOL, assert_close, assert_lse_close, build, note, W_name

pytestmark = pytest.mark.gpu

QMX = kvq.SPLIT_Q_MXFP8
WHOLE = kvq.SPLIT_WRITE_WHOLE_UNITS


def oracle_qmx(bl, seq_lens=None, pool=None):
    c = bl.case
    return OA.attention_ref(bl.geo, bl.pool_ref if pool is None else pool, W.bf16_bits(c.q), c.block_table,
                            c.seq_lens if seq_lens is None else seq_lens, c.softmax_scale, c.n_q, c.k_scale,
                            c.v_scale, q_mxfp8=True)


def run_qmx(bl, nwg=0, flags=WHOLE):
    c = bl.case
    q = c.q.cuda()
    ws = kvq.alloc_workspace(kvq.workspace_size(bl.desc, c.B, c.n_q, c.H_q, c.max_pages, nwg))
    ws.fill_(0xFF)
    out = torch.full((c.B, c.n_q, c.H_q, c.D), float("nan"), device="cuda")
    lse = torch.full((c.B, c.n_q, c.H_q), float("nan"), device="cuda")
    note("query-mxfp8 split", W_name(c), "nwg", nwg, "flags", flags)
    kvq.decode_split(bl.desc, bl.pool_gpu, q, bl.bt, bl.sl, c.softmax_scale, ws, num_workgroups=nwg,
                     flags=flags | QMX, out=out, lse=lse)
    kvq.decode_combine(bl.desc, c.B, c.n_q, c.H_q, c.max_pages, bl.sl, ws, out, lse, num_workgroups=nwg,
                       flags=flags | QMX)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy()


# (config, B, lengths): head_dim 128 with 4 query tokens (MHA), and head_dim
# 256 with 6 query heads per kv head
CASES = [
    (5, 4, [700, 260, 128, 3]),
    (2, 3, [1200, 65, 333]),
]


@pytest.mark.parametrize("cfg,B,lens", CASES)
def test_qmx_decode_matches_oracle_mode(cfg, B, lens):
    c = W.make_case(cfg, "MXFP8", device="cpu", B=B, lengths=lens)
    bl = build(c)
    out, lse = run_qmx(bl)
    ref, ref_lse = oracle_qmx(bl)
    assert_close(out, ref, "query-mxfp8 " + W_name(c))
    assert_lse_close(lse, ref_lse, "query-mxfp8 " + W_name(c))


@pytest.mark.parametrize("cfg", [5, 2])
def test_qmx_edge_lengths(cfg):
    lens = [0, 1, 15, 16, 17, 63, 64, 65, 127, 128, 129, 3]
    c = W.make_case(cfg, "MXFP8", device="cpu", B=len(lens), lengths=lens)
    bl = build(c)
    out, lse = run_qmx(bl)
    ref, ref_lse = oracle_qmx(bl)
    assert_close(out, ref, "query-mxfp8 edges " + W_name(c))
    assert_lse_close(lse, ref_lse, "query-mxfp8 edges " + W_name(c))
    assert np.all(out[0] == 0) and np.all(np.isneginf(lse[0]))


@pytest.mark.parametrize("cfg", [5, 2])
def test_qmx_follows_the_rounded_query(cfg):
    """The mode's attention differs from the plain one by far more than the
    tolerance (3-bit mantissas on q), and the kernel follows the mode's."""
    c = W.make_case(cfg, "MXFP8", device="cpu", B=2, lengths=[900, 301])
    bl = build(c)
    out, lse = run_qmx(bl)
    ref, ref_lse = oracle_qmx(bl)
    plain, _ = OA.attention_ref(bl.geo, bl.pool_ref, W.bf16_bits(c.q), c.block_table, c.seq_lens, c.softmax_scale,
                                c.n_q, c.k_scale, c.v_scale)
    assert np.any(np.abs(plain - ref) > 10 * (ATOL + RTOL * np.abs(ref))), "the case must tell the modes apart"
    assert_close(out, ref, "query-mxfp8 " + W_name(c))
    assert_lse_close(lse, ref_lse, "query-mxfp8 " + W_name(c))


def instruction_bound(bl, ref):
    """Extra error the block-scaled fp8 MFMA may add.  Measured on the
    instruction: within each run of 8 consecutive k (here 8 consecutive
    head_dim values) the products are aligned to the largest one's exponent
    E and summed with bits down to 2^(E - 13), smaller bits of each product
    dropped; so a run's sum is off by less than 7 * 2^-13 of its largest
    product.  Taken twice over (2^-9 per run) as the score error bound eps
    (natural-log units), a softmax moves each weight by a factor within
    e^(+-2 eps), so out moves by at most (e^(2 eps) - 1) max_t |v_t - out|
    and lse by eps."""
    c = bl.case
    q = OA.quantize_query_mxfp8(c.q.float().numpy().astype(np.float64))  # bf16 values, exact
    G = c.H_q // c.H_kv
    bo = np.zeros(ref.shape)
    bl_ = np.zeros(ref.shape[:3])
    for b in range(c.B):
        L = int(c.seq_lens[b])
        t = np.arange(L)
        slots = c.block_table[b][t // c.P].astype(np.int64) * c.P + t % c.P
        for h in range(c.H_kv):
            K, V = OA.decode_slots(bl.geo, bl.pool_ref, slots, h, c.k_scale, c.v_scale)
            for i in range(c.n_q):
                p = L - c.n_q + i
                if p < 0:
                    continue
                for j in range(G):
                    hq = h * G + j
                    prod = np.abs(q[b, i, hq][None, :] * K[:p + 1])            # [tokens, D]
                    runmax = prod.reshape(p + 1, c.D // 8, 8).max(axis=-1)      # [tokens, D / 8]
                    eps = c.softmax_scale * 2.0 ** -9 * runmax.sum(axis=-1).max()
                    spread = np.abs(V[:p + 1] - ref[b, i, hq][None, :]).max(axis=0)
                    bo[b, i, hq] = np.expm1(2 * eps) * spread
                    bl_[b, i, hq] = eps
    return bo, bl_


@pytest.mark.parametrize("cfg", [5, 2])
def test_qmx_dominant_elements_within_the_instruction_bound(cfg):
    """Query rows with one large element per 32-value group (and groups
    scaled by different powers of two): products of very different sizes
    share runs of 8, where the instruction drops low bits.  The kernel stays
    within the tolerance plus the bound those dropped bits allow, and the
    case still tells the mode's attention from the plain one."""
    c = W.make_case(cfg, "MXFP8", device="cpu", B=2, lengths=[900, 301])
    shape = c.q.shape
    gshape = shape[:-1] + (c.D // 32, 1)
    gen = torch.Generator().manual_seed(9)
    qg = c.q.float().reshape(shape[:-1] + (c.D // 32, 32))
    qg = qg * torch.exp2(torch.randint(-3, 4, gshape, generator=gen).float())
    qg.scatter_(-1, torch.randint(0, 32, gshape, generator=gen), 60.0)
    c.q = qg.reshape(shape).to(torch.bfloat16)
    c.softmax_scale = 1.0 / 16.0
    bl = build(c)
    out, lse = run_qmx(bl)
    ref, ref_lse = oracle_qmx(bl)
    plain, _ = OA.attention_ref(bl.geo, bl.pool_ref, W.bf16_bits(c.q), c.block_table, c.seq_lens, c.softmax_scale,
                                c.n_q, c.k_scale, c.v_scale)
    assert np.any(np.abs(plain - ref) > 10 * (ATOL + RTOL * np.abs(ref))), "the case must tell the modes apart"
    bo, bls = instruction_bound(bl, ref)
    err = np.abs(out - ref)
    bad = err > ATOL + RTOL * np.abs(ref) + bo
    assert not np.any(bad), "query-mxfp8 dominant elements: %d out of bound, max err %.3g" % (bad.sum(), err.max())
    fin = np.isfinite(ref_lse)
    assert np.all(np.abs(lse[fin] - ref_lse[fin]) <= 1e-3 + 1e-4 * np.abs(ref_lse[fin]) + bls[fin])


@pytest.mark.parametrize("cfg", [5, 2])
def test_qmx_workgroup_sweep(cfg):
    c = W.make_case(cfg, "MXFP8", device="cpu", B=3, lengths=[1100, 450, 77])
    bl = build(c)
    ref, ref_lse = oracle_qmx(bl)
    for nwg in (1, 3, 64, 333, 0):
        for flags in (0, WHOLE):
            out, lse = run_qmx(bl, nwg, flags)
            assert_close(out, ref, "query-mxfp8 nwg=%d flags=%d" % (nwg, flags))
            assert_lse_close(lse, ref_lse, "query-mxfp8 nwg=%d flags=%d" % (nwg, flags))


@pytest.mark.parametrize("cfg,lens", [(5, [700, 258, 124, 2]), (2, [1199, 64, 14])])
def test_qmx_fused_step(cfg, lens):
    """The fused step in the mode: the pool gets the oracle's bytes for the
    new tokens and the output is the mode's attention over the new cache."""
    n_new = W.CONFIGS[cfg]["n_q"]
    c = W.make_case(cfg, "MXFP8", device="cpu", B=len(lens), lengths=lens, reserve=n_new)
    bl = build(c)
    k, v, slots = W.append_chunk(c, n_new)
    sl_new = torch.as_tensor(c.seq_lens + n_new, dtype=torch.int32, device="cuda")
    q = c.q.cuda()
    B, n_q, H_q, D = q.shape
    pool = bl.pool_gpu.clone()
    ws = kvq.alloc_workspace(kvq.workspace_size(bl.desc, B, n_q, H_q, c.max_pages, 0))
    out = torch.full(q.shape, float("nan"), device="cuda")
    lse = torch.full(q.shape[:3], float("nan"), device="cuda")
    note("query-mxfp8 fused step", W_name(c))
    kvq.decode_step_split(bl.desc, pool, k.view(B, n_q, c.H_kv, D).cuda(), v.view(B, n_q, c.H_kv, D).cuda(), q,
                          bl.bt, sl_new, c.softmax_scale, ws, flags=WHOLE | QMX, out=out, lse=lse)
    kvq.decode_combine(bl.desc, B, n_q, H_q, c.max_pages, sl_new, ws, out, lse, flags=WHOLE | QMX)
    torch.cuda.synchronize()
    ref_pool = bl.pool_ref.copy()
    OA.quantize_append(bl.geo, ref_pool, W.bf16_bits(k), W.bf16_bits(v), slots.numpy(), c.k_scale, c.v_scale)
    assert np.array_equal(pool.cpu().numpy(), ref_pool)
    ref, ref_lse = oracle_qmx(bl, seq_lens=sl_new.cpu().numpy(), pool=ref_pool)
    assert_close(out.cpu().numpy(), ref, "query-mxfp8 fused step " + W_name(c))
    assert_lse_close(lse.cpu().numpy(), ref_lse, "query-mxfp8 fused step " + W_name(c))
