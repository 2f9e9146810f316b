"""kvq_decode_attention_noalloc (the entry point for callers that cannot
allocate: its workspace is the library's own device array) gives, through
the C ABI, exactly what kvq_decode_attention gives with a caller-owned
workspace, on two calls in a row (the second smaller, so it runs over what
the first left in the array), and refuses a problem too large for the array
without launching anything."""

import numpy as np
import pytest
import torch

import decode_attention_quant_amd as kvq
import workloads as W
from _gpu_common import assert_close, assert_lse_close, build, note, oracle_attention, W_name

pytestmark = pytest.mark.gpu


def _both(bl):
    c = bl.case
    q = c.q.cuda()
    res = []
    for noalloc in (False, True):
        out = torch.full((c.B, c.n_q, c.H_q, c.D), float("nan"), device="cuda")
        lse = torch.full((c.B, c.n_q, c.H_q), float("nan"), device="cuda")
        note("noalloc" if noalloc else "workspace", W_name(c))
        if noalloc:
            kvq.decode_attention_noalloc(bl.desc, bl.pool_gpu, q, bl.bt, bl.sl, c.softmax_scale, out, lse)
        else:
            ws = kvq.alloc_workspace(kvq.workspace_size(bl.desc, c.B, c.n_q, c.H_q, c.max_pages))
            ws.fill_(0x7F)
            kvq.decode_attention(bl.desc, bl.pool_gpu, q, bl.bt, bl.sl, c.softmax_scale, out=out, lse=lse,
                                 workspace=ws)
        torch.cuda.synchronize()
        res.append((out.cpu().numpy(), lse.cpu().numpy()))
    return res


@pytest.mark.parametrize("fmt,cfg,first,second", [
    ("K8V4", 4, [3000, 700, 65, 1290], [400, 17]),
    ("MXFP8", 5, [1500, 300, 129], [260]),
    ("NVFP4_G16", 3, [4100, 900], [77, 2]),
])
def test_noalloc_equals_decode_attention_twice(fmt, cfg, first, second):
    for lens in (first, second):
        c = W.make_case(cfg, fmt, device="cpu", B=len(lens), lengths=lens)
        bl = build(c)
        (o1, l1), (o2, l2) = _both(bl)
        assert np.array_equal(o1.view(np.uint32), o2.view(np.uint32)), "out differs " + W_name(c)
        assert np.array_equal(l1.view(np.uint32), l2.view(np.uint32)), "lse differs " + W_name(c)
        ref, ref_lse = oracle_attention(bl)
        assert_close(o2, ref, "noalloc " + W_name(c))
        assert_lse_close(l2, ref_lse, "noalloc " + W_name(c))


def test_noalloc_refuses_a_workspace_beyond_the_array():
    """4096 MHA sequences at 32 heads and 4 query tokens plan over 256 MB of
    partials, past the 64 MiB array: refused, nothing written."""
    B = 4096
    d = kvq.desc("MXFP8", 128, 128, 32, 64)
    need = kvq.workspace_size(d, B, 4, 32, 64)
    assert need > kvq.NOALLOC_SCRATCH_BYTES
    pool = kvq.alloc_pool(d)
    q = torch.zeros((B, 4, 32, 128), dtype=torch.bfloat16, device="cuda")
    bt = torch.zeros((B, 64), dtype=torch.int32, device="cuda")
    sl = torch.full((B,), 100, dtype=torch.int32, device="cuda")
    out = torch.full((B, 4, 32, 128), 3.0, device="cuda")
    note("noalloc refusal")
    with pytest.raises(kvq.KvqError) as e:
        kvq.decode_attention_noalloc(d, pool, q, bt, sl, 0.1, out)
    assert e.value.status == 3
    torch.cuda.synchronize()
    assert bool((out == 3.0).all())
