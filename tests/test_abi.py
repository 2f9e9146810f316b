"""The C ABI: library loads, exports what include/kvq.h declares, and rejects
bad arguments on the host before any HIP call (CPU only; no kernel runs)."""

import ctypes
import os
import re

import pytest

import decode_attention_quant_amd as kvq
from oracle import layout as Lo

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvq.h")

pytestmark = pytest.mark.skipif(not os.path.exists(kvq.LIB_PATH), reason="libkvq.so not built")


def header_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^(?:kvq_status|const char\*)\s+(kvq_\w+)\s*\(", text, re.M)))


def test_header_declares_the_boundary():
    fns = header_functions()
    for name in ("kvq_quantize_append", "kvq_decode_attention", "kvq_dequant_page"):
        assert name in fns
    assert set(fns) == set(kvq.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = kvq.library()
    for name in header_functions():
        assert hasattr(lib, name), name


def test_status_strings():
    lib = kvq.library()
    for s in range(5):
        assert lib.kvq_status_string(s)
    assert lib.kvq_status_string(99) == b"unknown status"


@pytest.mark.parametrize("fmt", range(8))
@pytest.mark.parametrize("D,P", [(128, 64), (256, 64), (256, 128), (128, 128)])
def test_page_bytes_match_the_oracle_layout(fmt, D, P):
    d = kvq.desc(fmt, D, P, 3, 10, 0.5, 0.5)
    rotated = fmt in (1, 3, 4, 7)
    if rotated and D != 256:
        with pytest.raises(kvq.KvqError) as e:
            kvq.page_bytes(d)
        assert e.value.status == 2
        return
    assert kvq.page_bytes(d) == Lo.Geometry(fmt, D, P, 3).page_bytes


def _status(fn, *args):
    return getattr(kvq.library(), fn)(*args)


def test_desc_validation():
    out = ctypes.c_size_t()
    bad = [
        (kvq.desc(8, 256, 64, 2, 4), 1),       # unknown format
        (kvq.desc(-1, 256, 64, 2, 4), 1),
        (kvq.desc(0, 256, 64, 0, 4), 1),       # no kv heads
        (kvq.desc(0, 256, 64, 2, 0), 1),       # no pages
        (kvq.desc(0, 192, 64, 2, 4), 2),       # head_dim
        (kvq.desc(0, 256, 32, 2, 4), 2),       # page size
        (kvq.desc(3, 128, 64, 2, 4), 2),       # rotation needs 256
        (kvq.desc(6, 256, 64, 2, 4, 0.0, 1.0), 1),            # tensor scale must be > 0
        (kvq.desc(6, 256, 64, 2, 4, 1.0, float("inf")), 1),
        (kvq.desc(6, 256, 64, 2, 4, float("nan"), 1.0), 1),
        (kvq.desc(3, 256, 64, 2, 4, 0.0, 1.0), 1),            # two-level NVFP4: both scales > 0
        (kvq.desc(3, 256, 64, 2, 4, 1.0, -2.0), 1),
        (kvq.desc(4, 256, 64, 2, 4, 1.0, float("nan")), 1),   # K8V4: its NVFP4 V scale
    ]
    for d, want in bad:
        assert _status("kvq_page_bytes", ctypes.byref(d), ctypes.byref(out)) == want
    assert _status("kvq_page_bytes", None, ctypes.byref(out)) == 1
    # scales a format does not use are ignored (K8V4's FP8-row K, FP8-row)
    for d in (kvq.desc(4, 256, 64, 2, 4, -5.0, 1.0), kvq.desc(2, 256, 64, 2, 4, 0.0, float("nan"))):
        assert _status("kvq_page_bytes", ctypes.byref(d), ctypes.byref(out)) == 0
    d = kvq.desc(0, 256, 64, 2, 4)
    assert _status("kvq_page_bytes", ctypes.byref(d), None) == 1


def test_append_validation_enqueues_nothing():
    d = kvq.desc(2, 256, 64, 2, 4)
    P = ctypes.c_void_p
    ok = P(0x10000)
    # zero tokens is a no-op that succeeds without touching the GPU
    assert _status("kvq_quantize_append", ctypes.byref(d), None, None, None, 0, None, None) == 0
    assert _status("kvq_quantize_append", ctypes.byref(d), ok, ok, ok, -1, ok, None) == 1
    assert _status("kvq_quantize_append", ctypes.byref(d), None, ok, ok, 5, ok, None) == 1
    assert _status("kvq_quantize_append", ctypes.byref(d), ok, ok, ok, 5, None, None) == 1
    assert _status("kvq_quantize_append", ctypes.byref(d), P(0x10040), ok, ok, 5, ok, None) == 1  # pool alignment
    assert _status("kvq_quantize_append", ctypes.byref(d), ok, P(0x10008), ok, 5, ok, None) == 1  # k alignment


def test_workspace_size_with_forced_workgroups():
    d = kvq.desc(1, 256, 64, 4, 100)
    sz = ctypes.c_size_t()
    assert _status("kvq_decode_workspace_size_for", ctypes.byref(d), 3, 1, 24, 10, 7, ctypes.byref(sz)) == 0
    units, nwg, R = 3 * 4, 7, 6
    slots = units + nwg
    a256 = lambda n: (n + 255) // 256 * 256
    assert sz.value == a256(4 * 4) + a256(slots * R * 2 * 4) + slots * R * 256 * 4
    bad = [(3, 0, 24, 10, 4), (3, 1, 0, 10, 4), (3, 1, 25, 10, 4), (-1, 1, 24, 10, 4), (3, 1, 24, 0, 4),
           (3, 1, 24, 10, -2)]
    for args in bad:
        assert _status("kvq_decode_workspace_size_for", ctypes.byref(d), *args, ctypes.byref(sz)) == 1, args
    # too many rows per kv head, or too large a batch
    assert _status("kvq_decode_workspace_size_for", ctypes.byref(d), 1, 64, 4 * 32, 10, 4, ctypes.byref(sz)) == 2
    assert _status("kvq_decode_workspace_size_for", ctypes.byref(d), 5000, 1, 24, 10, 4, ctypes.byref(sz)) == 2
    # the planned form validates the same arguments before asking the device
    for args in [a[:4] for a in bad if a[4] >= 0]:
        assert _status("kvq_decode_workspace_size", ctypes.byref(d), *args, ctypes.byref(sz)) == 1, args
    assert _status("kvq_decode_workspace_size", ctypes.byref(d), 3, 1, 24, 10, None) == 1


# The calls of the boundary as the survey of the pages lists them: name ->
# parameter types in order (names of parameters are free).
SURVEY_SIGNATURES = {
    "kvq_page_bytes": ["const kvq_cache_desc*", "size_t*"],
    "kvq_quantize_append": ["const kvq_cache_desc*", "void*", "const void*", "const void*", "int64_t",
                            "const int32_t*", "hipStream_t"],
    "kvq_decode_workspace_size": ["const kvq_cache_desc*", "int32_t", "int32_t", "int32_t", "int32_t", "size_t*"],
    "kvq_decode_attention": ["const kvq_cache_desc*", "const void*", "const void*", "int32_t", "int32_t", "int32_t",
                             "const int32_t*", "int32_t", "const int32_t*", "float", "float*", "float*", "void*",
                             "size_t", "hipStream_t"],
    "kvq_dequant_page": ["const kvq_cache_desc*", "const void*", "int64_t", "int32_t", "float*", "float*",
                         "hipStream_t"],
    "kvq_status_string": ["kvq_status"],
}


def _header_signatures():
    text = re.sub(r"/\*.*?\*/", " ", open(HEADER).read(), flags=re.S)
    sigs = {}
    for m in re.finditer(r"(kvq_status|const char\*)\s+(kvq_\w+)\s*\(([^)]*)\)\s*;", text):
        params = []
        for p in m.group(3).split(","):
            p = " ".join(p.split())
            p = re.sub(r"\s*\*\s*", "* ", p).strip()
            toks = p.split(" ")
            params.append(" ".join(toks[:-1]).replace(" *", "*").strip())
        sigs[m.group(2)] = params
    return sigs


def test_noalloc_scratch_size_matches_the_header():
    m = re.search(r"#define KVQ_NOALLOC_SCRATCH_BYTES \((\d+) << (\d+)\)", open(HEADER).read())
    assert m and int(m.group(1)) << int(m.group(2)) == kvq.NOALLOC_SCRATCH_BYTES


def test_boundary_calls_have_the_survey_signatures():
    sigs = _header_signatures()
    for name, params in SURVEY_SIGNATURES.items():
        assert name in sigs, name
        assert sigs[name] == params, (name, sigs[name])


def test_decode_validation_enqueues_nothing():
    d = kvq.desc(2, 256, 64, 4, 100)
    P = ctypes.c_void_p
    ok = P(0x100000)
    lib = kvq.library()
    args = dict(pool=ok, q=ok, B=2, nq=1, Hq=24, bt=ok, mp=10, sl=ok, scale=0.0625, out=ok, lse=None, ws=ok,
                wsb=1 << 30)

    def call(**kw):
        a = dict(args, **kw)
        return lib.kvq_decode_split(ctypes.byref(d), a["pool"], a["q"], a["B"], a["nq"], a["Hq"], a["bt"], a["mp"],
                                    a["sl"], a["scale"], 4, a.get("flags", 0), a["out"], a["lse"], a["ws"],
                                    a["wsb"], None)

    assert call(B=0) == 0  # empty batch: nothing to do
    assert call(pool=None) == 1
    assert call(q=None) == 1
    assert call(bt=None) == 1
    assert call(sl=None) == 1
    assert call(ws=None) == 1
    assert call(q=P(0x100004)) == 1
    assert call(ws=P(0x100080)) == 1   # workspace must be 256-byte aligned
    assert call(pool=P(0x100040)) == 1  # pool must be 128-byte aligned
    assert call(scale=float("nan")) == 1
    assert call(wsb=100) == 3
    assert call(Hq=22) == 1            # not a multiple of H_kv
    assert call(flags=4) == 1          # unknown flag
    assert call(flags=2) == 2          # the query-MXFP8 mode needs an MXFP8 cache
    assert call(flags=3) == 2
    mx = kvq.desc(5, 128, 128, 32, 100)
    assert lib.kvq_decode_split(ctypes.byref(mx), ok, ok, 0, 4, 32, ok, 10, ok, 0.1, 4, 2, None, None, ok,
                                1 << 30, None) == 0  # accepted (empty batch: nothing to do)
    assert lib.kvq_decode_combine(ctypes.byref(mx), 0, 4, 32, 10, ok, 4, 3, ok, 1 << 30, ok, None, None) == 0
    assert lib.kvq_decode_combine(ctypes.byref(mx), 0, 4, 32, 10, ok, 4, 4, ok, 1 << 30, ok, None, None) == 1
    assert call(flags=1, out=None) == 1  # finishing whole units needs out
    bad = kvq.desc(3, 128, 64, 4, 100)
    assert lib.kvq_decode_split(ctypes.byref(bad), ok, ok, 2, 1, 24, ok, 10, ok, 0.1, 4, 0, None, None, ok,
                                1 << 30, None) == 2


def test_dequant_validation():
    d = kvq.desc(0, 256, 64, 2, 4)
    P = ctypes.c_void_p
    ok = P(0x100000)
    lib = kvq.library()
    assert lib.kvq_dequant_page(ctypes.byref(d), ok, 4, 1, ok, ok, None) == 1    # page out of range
    assert lib.kvq_dequant_page(ctypes.byref(d), ok, -1, 1, ok, ok, None) == 1
    assert lib.kvq_dequant_page(ctypes.byref(d), ok, 0, 2, ok, ok, None) == 1    # unknown flag
    assert lib.kvq_dequant_page(ctypes.byref(d), None, 0, 1, ok, ok, None) == 1
    assert lib.kvq_dequant_page(ctypes.byref(d), ok, 0, 1, P(0x100004), ok, None) == 1


# ---- libkvq_probe.so: the measurement kernels' C ABI (kvq_probe.h)

PROBE_HEADER = os.path.join(ROOT, "include", "kvq_probe.h")


def test_probe_header_matches_exports():
    from decode_attention_quant_amd import probe
    fns = sorted(set(re.findall(r"^int\s+(kvq_probe_\w+)\s*\(", open(PROBE_HEADER).read(), re.M)))
    assert fns == sorted(probe.EXPORTS)
    lib = probe.library()
    for name in fns:
        assert hasattr(lib, name), name


def test_probe_rejects_bad_arguments_on_the_host():
    from decode_attention_quant_amd import probe
    lib = probe.library()
    fake = ctypes.c_void_p(1 << 20)  # never dereferenced: validation fails first
    assert lib.kvq_probe_read(None, 1024, fake, None) == 1
    assert lib.kvq_probe_read(fake, 1000, fake, None) == 1          # not whole 1 KB chunks
    assert lib.kvq_probe_read(ctypes.c_void_p((1 << 20) + 8), 1024, fake, None) == 1  # misaligned
    assert lib.kvq_probe_read(fake, 1024, None, None) == 1
    assert lib.kvq_probe_read_stream(None, 1024, fake, None) == 1
    assert lib.kvq_probe_read_stream(fake, 1000, fake, None) == 1
    assert lib.kvq_probe_copy(fake, fake, 24, None) == 1            # not whole 16 B words
    assert lib.kvq_probe_copy(None, fake, 32, None) == 1
    assert lib.kvq_probe_read(fake, 0, fake, None) == 0             # empty: nothing to do
    assert lib.kvq_probe_copy(fake, fake, 0, None) == 0


def test_decode_step_validation_enqueues_nothing():
    """The fused step's own checks come before any HIP call."""
    d = kvq.desc(3, 256, 64, 4, 100)
    P = ctypes.c_void_p
    ok = P(0x100000)
    lib = kvq.library()

    def call(k=ok, v=ok, B=2, nq=1, Hq=24, pool=ok):
        return lib.kvq_decode_step(ctypes.byref(d), pool, k, v, ok, B, nq, Hq, ok, 10, ok, 0.0625, ok, None, ok,
                                   1 << 30, None)

    assert call(B=0) == 0                   # empty batch: nothing to do
    assert call(k=None) == 1
    assert call(v=None) == 1
    assert call(k=P(0x100008)) == 1         # 16-byte alignment of the new rows
    assert call(nq=3) == 2                  # G * n_q = 18 rows: more than one row tile
    assert call(Hq=22) == 1                 # not a multiple of H_kv
    assert call(pool=None, nq=1) == 1


def test_prefill_validation_enqueues_nothing():
    d = kvq.desc(4, 256, 64, 4, 100)
    P = ctypes.c_void_p
    ok = P(0x100000)
    lib = kvq.library()

    def call(pool=ok, q=ok, B=2, nq=37, Hq=24, bt=ok, sl=ok, out=ok, scale=0.0625):
        return lib.kvq_prefill_attention(ctypes.byref(d), pool, q, B, nq, Hq, bt, 10, sl, scale, out, None, None)

    assert call(B=0) == 0
    assert call(pool=None) == 1
    assert call(q=None) == 1
    assert call(bt=None) == 1
    assert call(sl=None) == 1
    assert call(out=None) == 1
    assert call(q=P(0x100008)) == 1
    assert call(out=P(0x100004)) == 1
    assert call(nq=0) == 1
    assert call(Hq=22) == 1
    assert call(scale=float("inf")) == 1
    bad = kvq.desc(3, 128, 64, 4, 100)  # NVFP4 needs head_dim 256
    assert lib.kvq_prefill_attention(ctypes.byref(bad), ok, ok, 2, 4, 24, ok, 10, ok, 0.1, ok, None, None) == 2
