"""Shared helpers of the GPU parity tests: build the same cache on the GPU
(through the C ABI) and in the oracle (on the CPU) from one seeded draw."""

import sys

import numpy as np
import torch

import decode_attention_quant_amd as kvq
import workloads as W
from oracle import attention as OA, layout as OL

ATOL, RTOL = 1e-3, 2e-3   # |gpu - ref| <= ATOL + RTOL * |ref| (fp64 oracle)


def note(*a):
    """Name the case before each GPU step so a failure log says which one."""
    print("[gpu-case]", *a, flush=True)
    sys.stdout.flush()


def require_gpu():
    if not torch.cuda.is_available():
        raise RuntimeError("a GPU test ran without a GPU")
    kvq.library()  # raises if the HIP library is missing: no fallback exists


class Built:
    """One workload encoded by both sides."""

    def __init__(self, case, geo, desc, pool_gpu, pool_ref, bt, sl):
        self.case, self.geo, self.desc = case, geo, desc
        self.pool_gpu, self.pool_ref = pool_gpu, pool_ref
        self.bt, self.sl = bt, sl


def build(case, fill=0xFF, oracle=True):
    require_gpu()
    geo = OL.Geometry(case.fmt, case.D, case.P, case.H_kv)
    d = kvq.desc(case.fmt, case.D, case.P, case.H_kv, case.num_pages, case.k_scale, case.v_scale)
    pool = kvq.alloc_pool(d, fill=fill)
    note("append", W_name(case), "T=%d" % case.k.shape[0])
    kvq.quantize_append(d, pool, case.k.cuda(), case.v.cuda(), case.slot_mapping.cuda())
    torch.cuda.synchronize()
    ref = None
    if oracle:
        ref = np.full(case.num_pages * geo.page_bytes, fill, dtype=np.uint8)
        OA.quantize_append(geo, ref, W.bf16_bits(case.k), W.bf16_bits(case.v),
                           case.slot_mapping.cpu().numpy(), case.k_scale, case.v_scale)
    bt = torch.as_tensor(case.block_table, device="cuda")
    sl = torch.as_tensor(case.seq_lens, device="cuda")
    return Built(case, geo, d, pool, ref, bt, sl)


def W_name(case):
    return "cfg=%s fmt=%s B=%d D=%d P=%d Hq=%d Hkv=%d nq=%d lens=%s" % (
        case.config, kvq.FORMAT_NAMES[case.fmt], case.B, case.D, case.P, case.H_q, case.H_kv, case.n_q,
        list(case.seq_lens[:8]))


def oracle_attention(bl, only=None):
    c = bl.case
    return OA.attention_ref(bl.geo, bl.pool_ref, W.bf16_bits(c.q), c.block_table, c.seq_lens, c.softmax_scale,
                            c.n_q, c.k_scale, c.v_scale, only=only)


def assert_close(got, ref, what):
    got = np.asarray(got, dtype=np.float64)
    bad = np.abs(got - ref) > ATOL + RTOL * np.abs(ref)
    ok_nan = np.isnan(ref)
    bad &= ~ok_nan
    if np.any(bad):
        idx = np.argwhere(bad)[:5]
        raise AssertionError("%s: %d of %d elements out of tolerance, e.g. %s got %s ref %s; max err %.3g" % (
            what, int(bad.sum()), bad.size, idx.tolist(), got[tuple(idx.T)], ref[tuple(idx.T)],
            np.nanmax(np.abs(got - ref))))


def assert_lse_close(got, ref, what):
    got = np.asarray(got, dtype=np.float64)
    inf = np.isneginf(ref)
    assert np.array_equal(np.isneginf(got), inf), what + ": -inf pattern"
    fin = ~inf & ~np.isnan(ref)
    err = np.abs(got[fin] - ref[fin])
    assert np.all(err <= 1e-3 + 1e-4 * np.abs(ref[fin])), "%s: lse max err %.3g" % (what, err.max() if err.size else 0)
