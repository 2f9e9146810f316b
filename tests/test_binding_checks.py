"""The Python binding checks every tensor's dtype, shape, contiguity and
byte size against the cache descriptor and against each other before any
pointer crosses the boundary (CPU only: the tensors here live on the host,
so a call that got past the checks would stop at the device check, and no
kernel is ever launched)."""

import os

import pytest
import torch

import decode_attention_quant_amd as kvq

pytestmark = pytest.mark.skipif(not os.path.exists(kvq.LIB_PATH), reason="libkvq.so not built")

B, NQ, HQ, HKV, D, P, PAGES, MAXP = 2, 1, 8, 2, 256, 64, 6, 3


def _desc(fmt="FP8_ROW"):
    return kvq.desc(fmt, D, P, HKV, PAGES)


def _good():
    d = _desc()
    return dict(
        d=d,
        pool=torch.zeros(kvq.page_bytes(d) * PAGES, dtype=torch.uint8),
        q=torch.zeros((B, NQ, HQ, D), dtype=torch.bfloat16),
        bt=torch.zeros((B, MAXP), dtype=torch.int32),
        sl=torch.zeros((B,), dtype=torch.int32),
        out=torch.zeros((B, NQ, HQ, D), dtype=torch.float32),
        lse=torch.zeros((B, NQ, HQ), dtype=torch.float32),
        ws=torch.zeros((1 << 20,), dtype=torch.uint8),
        k=torch.zeros((5, HKV, D), dtype=torch.bfloat16),
        slots=torch.zeros((5,), dtype=torch.int32),
        k_new=torch.zeros((B, NQ, HKV, D), dtype=torch.bfloat16),
    )


def _decode(g, **over):
    a = dict(g, **over)
    kvq.decode_attention(a["d"], a["pool"], a["q"], a["bt"], a["sl"], 0.0625, out=a["out"], lse=a["lse"],
                         workspace=a["ws"])


def _raises(fn, what):
    with pytest.raises(ValueError) as e:
        fn()
    assert what in str(e.value), str(e.value)


def test_well_formed_host_tensors_stop_at_the_device_check():
    g = _good()
    _raises(lambda: _decode(g), "must be a CUDA tensor")
    _raises(lambda: kvq.quantize_append(g["d"], g["pool"], g["k"], g["k"], g["slots"]), "must be a CUDA tensor")


@pytest.mark.parametrize("name,bad,what", [
    ("q", torch.zeros((B, NQ, HQ, 128), dtype=torch.bfloat16), "head_dim"),
    ("q", torch.zeros((B, NQ, 7, D), dtype=torch.bfloat16), "not a multiple of num_kv_heads"),
    ("q", torch.zeros((B, NQ, HQ, D), dtype=torch.float16), "q must be torch.bfloat16"),
    ("q", torch.zeros((B, HQ, D), dtype=torch.bfloat16), "4-D"),
    ("q", torch.zeros((B, NQ, D, HQ), dtype=torch.bfloat16).transpose(2, 3), "contiguous"),
    ("bt", torch.zeros((B + 1, MAXP), dtype=torch.int32), "block_table must have shape"),
    ("bt", torch.zeros((B, MAXP), dtype=torch.int64), "block_table must be torch.int32"),
    ("bt", torch.zeros((B * MAXP,), dtype=torch.int32), "2-D"),
    ("sl", torch.zeros((B + 3,), dtype=torch.int32), "seq_lens must have shape"),
    ("out", torch.zeros((B, NQ, HQ, D - 1), dtype=torch.float32), "out must have shape"),
    ("out", torch.zeros((B, NQ, HQ, D), dtype=torch.float16), "out must be torch.float32"),
    ("lse", torch.zeros((B, NQ, HQ + 1), dtype=torch.float32), "lse must have shape"),
    ("pool", torch.zeros((100,), dtype=torch.uint8), "pool holds"),
    ("pool", torch.zeros((10, 10), dtype=torch.uint8), "1-D uint8"),
    ("ws", torch.zeros((64,), dtype=torch.int32), "workspace must be torch.uint8"),
])
def test_decode_rejects_mismatched_tensors(name, bad, what):
    _raises(lambda: _decode(_good(), **{name: bad}), what)


def test_append_rejects_mismatched_tensors():
    g = _good()
    d, pool = g["d"], g["pool"]
    k = g["k"]
    _raises(lambda: kvq.quantize_append(d, pool, torch.zeros((5, HKV, 128), dtype=torch.bfloat16), k, g["slots"]),
            "k must have shape")
    _raises(lambda: kvq.quantize_append(d, pool, k, torch.zeros((4, HKV, D), dtype=torch.bfloat16), g["slots"]),
            "v must have shape")
    _raises(lambda: kvq.quantize_append(d, pool, k, k, torch.zeros((6,), dtype=torch.int32)),
            "slot_mapping must have shape")
    _raises(lambda: kvq.quantize_append(d, pool, k, k, g["slots"].long()), "slot_mapping must be torch.int32")
    _raises(lambda: kvq.quantize_append(d, pool[:-1], k, k, g["slots"]), "pool holds")


def test_step_rejects_mismatched_new_tokens():
    g = _good()
    args = (g["d"], g["pool"])
    bad = torch.zeros((B, NQ + 1, HKV, D), dtype=torch.bfloat16)
    _raises(lambda: kvq.decode_step(*args, bad, g["k_new"], g["q"], g["bt"], g["sl"], 0.0625, out=g["out"],
                                    workspace=g["ws"]), "k_new must have shape")
    _raises(lambda: kvq.decode_step(*args, g["k_new"], bad, g["q"], g["bt"], g["sl"], 0.0625, out=g["out"],
                                    workspace=g["ws"]), "v_new must have shape")
    _raises(lambda: kvq.decode_step_split(*args, g["k_new"], g["k_new"].float(), g["q"], g["bt"], g["sl"], 0.0625,
                                          g["ws"]), "v_new must be torch.bfloat16")


def test_phases_and_prefill_and_dequant_check_too():
    g = _good()
    d, pool = g["d"], g["pool"]
    _raises(lambda: kvq.decode_split(d, pool, g["q"], g["bt"][:1], g["sl"], 0.0625, g["ws"]),
            "block_table must have shape")
    _raises(lambda: kvq.decode_combine(d, B, NQ, HQ, MAXP, g["sl"], g["ws"], g["out"][:1]), "out must have shape")
    _raises(lambda: kvq.decode_combine(d, B, NQ, 7, MAXP, g["sl"], g["ws"], g["out"]), "not a multiple")
    _raises(lambda: kvq.prefill_attention(d, pool, g["q"][:, :, :, :128].contiguous(), g["bt"], g["sl"], 0.0625),
            "head_dim")
    _raises(lambda: kvq.dequant_page(d, pool, PAGES), "outside the pool")
    _raises(lambda: kvq.dequant_page(d, pool[:10], 0), "pool holds")
