"""GPU parity of chunked-prefill attention against the fp64 oracle.

A prefill chunk of n_q tokens is appended to each cached sequence (through
the write path on both sides), then every query of the chunk attends
causally over the whole cache.  The oracle's definition is the one decode
uses (query i at position L_b - n_q + i sees positions 0 .. that one), so
the same tolerance applies: |gpu - ref| <= 1e-3 + 2e-3 |ref|.
"""

import numpy as np
import pytest
import torch

import decode_attention_quant_amd as kvq
import workloads as W
from oracle import attention as OA
from _gpu_common import assert_close, assert_lse_close, build, note, W_name

pytestmark = pytest.mark.gpu


def prefill_case(cfg, fmt, lens, chunk):
    """A cache of `lens` tokens per sequence plus a `chunk`-token prefill chunk
    appended on both sides; returns (case, built, seq_lens after the chunk)."""
    c = W.make_case(cfg, fmt, device="cpu", B=len(lens), lengths=lens, n_q=chunk, reserve=chunk)
    bl = build(c)
    k, v, slots = W.append_chunk(c, chunk)
    note("prefill append", W_name(c), "chunk", chunk)
    kvq.quantize_append(bl.desc, bl.pool_gpu, k.cuda(), v.cuda(), slots.cuda())
    OA.quantize_append(bl.geo, bl.pool_ref, W.bf16_bits(k), W.bf16_bits(v), slots.numpy(), c.k_scale, c.v_scale)
    torch.cuda.synchronize()
    return c, bl, (c.seq_lens + chunk).astype(np.int32)


def run_prefill(c, bl, sl):
    q = c.q.cuda()
    out = torch.full(q.shape, float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device="cuda")
    note("prefill", W_name(c), "n_q", q.shape[1])
    kvq.prefill_attention(bl.desc, bl.pool_gpu, q, bl.bt, torch.as_tensor(sl, device="cuda"), c.softmax_scale,
                          out=out, lse=lse)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy()


def oracle(c, bl, sl):
    return OA.attention_ref(bl.geo, bl.pool_ref, W.bf16_bits(c.q), c.block_table, sl, c.softmax_scale, c.n_q,
                            c.k_scale, c.v_scale)


# (config, format, cached lengths, chunk): G * chunk rows per kv head span
# several row tiles (64 rows on the 16-row kernel, 128 on the 32-row one)
# with a ragged last one, and waves with no rows; chunks start mid-block
CASES = [
    (1, "BF16", [300], 37),
    (1, "FP8_ROW", [300], 37),
    (2, "INT8_G64", [300, 70], 45),
    (2, "FP8_ROW", [300, 70], 45),
    (2, "FP8_TENSOR", [300, 70], 45),
    (3, "NVFP4_G16", [260, 33], 40),
    (4, "K8V4", [150, 400, 7], 29),
    (5, "MXFP8", [200, 61], 70),
    (5, "BF16", [200, 61], 70),
    (5, "FP8_ROW", [200, 61], 70),      # head_dim 128 on the 32-row kernel, two V buffers
    (5, "FP8_TENSOR", [131, 60], 67),
    (3, "MXFP4", [260, 33], 41),
]


@pytest.mark.parametrize("cfg,fmt,lens,chunk", CASES)
def test_prefill_matches_oracle(cfg, fmt, lens, chunk):
    c, bl, sl = prefill_case(cfg, fmt, lens, chunk)
    out, lse = run_prefill(c, bl, sl)
    ref, ref_lse = oracle(c, bl, sl)
    assert_close(out, ref, "prefill " + W_name(c))
    assert_lse_close(lse, ref_lse, "prefill " + W_name(c))


@pytest.mark.parametrize("cfg,fmt", [(3, "NVFP4_G16"), (4, "K8V4"), (1, "BF16")])
def test_prefill_short_and_empty_sequences(cfg, fmt):
    """Sequences shorter than the chunk: early queries see nothing (out 0,
    lse -inf); an empty cache before the chunk; one sequence of length 0.
    NVFP4 runs the 16-row kernel, K8V4 and BF16 the 32-row one (where whole
    waves then see nothing in a step)."""
    c, bl, sl = prefill_case(cfg, fmt, [0, 5, 90], 24)
    sl = sl.copy()
    sl[1] = 10   # only the first 10 of sequence 1's 29 positions: queries 0 .. 13 see nothing
    sl[0] = 0    # sequence 0 has nothing at all
    out, lse = run_prefill(c, bl, sl)
    ref, ref_lse = oracle(c, bl, sl)
    assert_close(out, ref, "prefill short")
    assert_lse_close(lse, ref_lse, "prefill short")
    assert np.all(out[0] == 0) and np.all(np.isneginf(lse[0]))
    assert np.all(out[1, :14] == 0) and np.all(np.isneginf(lse[1, :14]))


@pytest.mark.parametrize("fmt,cfg", [("K8V4", 4), ("MXFP8", 5), ("INT8_G64", 2), ("MXFP4", 3)])
def test_prefill_agrees_with_decode(fmt, cfg):
    """Where both apply (few query tokens), prefill and decode compute the same
    attention.  They differ in how the blocks are grouped (decode's four waves
    each keep a running maximum over a quarter of the blocks), and P is
    rounded to f16 relative to that maximum, so they agree to the decode
    tolerance, not bit for bit."""
    chunk = 2
    c, bl, sl = prefill_case(cfg, fmt, [500, 129, 40], chunk)
    out, lse = run_prefill(c, bl, sl)
    q = c.q.cuda()
    dout = torch.empty(q.shape, dtype=torch.float32, device="cuda")
    dlse = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
    note("decode for comparison", W_name(c))
    kvq.decode_attention(bl.desc, bl.pool_gpu, q, bl.bt, torch.as_tensor(sl, device="cuda"), c.softmax_scale,
                         out=dout, lse=dlse)
    torch.cuda.synchronize()
    assert_close(out, dout.cpu().numpy().astype(np.float64), "prefill vs decode " + W_name(c))
    assert_lse_close(lse, dlse.cpu().numpy().astype(np.float64), "prefill vs decode " + W_name(c))
