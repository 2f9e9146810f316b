"""Benchmark: one decode step of the quantized paged-KV hot path on MI355X.

A step is the whole hot path over one batch: quantize-append of each
sequence's newest token (K and V of every kv head, through the codec and the
Hadamard rotation where the format has it), then split-K decode attention
over every cached page and the cross-split combine.  Inputs are resident in
HBM before timing starts, and before every timed step a 1 GiB read evicts
the L2 caches and the 256 MB MALL, so each step streams the cache from HBM
as it would between two layers of a model (``--no-flush`` times the steps
back to back instead).  By default every decode workload is timed, for each
of its kv-dtypes, and reported under ``per_workload``: tiny (1 x 1024, BF16
and FP8 row-256: a latency), batched (32 x U[8K, 32K] tokens, INT8-G64, FP8
row-256, per-tensor FP8), long (1 x 262144 tokens: NVFP4-G16, two-level
NVFP4, MXFP4), long8 (8 x 65536, NVFP4-G16), mixed (64 x logU[1K, 128K],
K8V4) and mtp (256 x 4096, 4 query tokens, MHA, MXFP8 plain and with the
query rounded to MXFP8).  The headline value is the batched decode's
INT8-G64 step (24 query / 4 KV heads, head_dim 256, 64-token pages).

The write path is measured on its own workload: one 2048-token prefill chunk
for each of 64 mixed-length sequences (log-uniform 1K-128K cached tokens,
chunks starting mid-page), K8V4 first, then the other formats at that shape.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload all|batched|long|...]

Prints one JSON line.  ``value`` is effective compressed-KV bandwidth:
sum_b H_kv * L_b * bytes_per_token / ms_per_step.  ``roofline`` prices the
dominant kernel (the split kernel) against the 8 TB/s HBM peak with its
average duration measured by HIP events on its own stream, next to the read
rate a plain streaming kernel reaches on the same device; its ``traffic``
comes from committed HBM byte counters, only while the kernel sources still
hash to what was profiled.  ``cpu_baseline`` times the CPU oracle on a
bounded sample of the same workload.

    python bench.py --summarize-counters FETCH_DIR WRITE_DIR BENCH_JSON [FETCH_DIR WRITE_DIR BENCH_JSON ...]

turns pairs of rocprofv3 --pmc runs of this script (FETCH_SIZE, then
WRITE_SIZE, each on one workload and format, with that run's JSON line) into
a list of traffic records: per-dispatch KiB of the split kernel, scaled by
what the same counters read for the probe's copy kernel of known size.
"""

import argparse
import gc
import csv
import glob
import hashlib
import json
import math
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import decode_attention_quant_amd as kvq  # noqa: E402
import workloads as W  # noqa: E402

HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense f16 / bf16 matrix peak
FLUSH_BYTES = 1 << 30          # read before each timed step: 4x the 256 MB MALL
RATE_BYTES = 4 << 30           # buffer of the streaming-rate measurement
COPY_BYTES = RATE_BYTES // 2   # bytes each way of the probe's copy
APPEND_CHUNK = 2048
APPEND_FORMATS = ["K8V4", "BF16", "INT8_G64", "FP8_ROW", "NVFP4_G16", "FP8_TENSOR", "NVFP4_G16/2L", "MXFP4"]
CSRC = os.path.join(ROOT, "decode_attention_quant_amd", "csrc")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_split_traffic.json")
METRIC = "decode-attn effective KV GB/s (% of HBM peak) per kv-dtype; quant-append tok/s"


class HipEvent:
    """A HIP timing event, created with hipEventDisableSystemFence: its
    record then skips the system-scope release (a writeback and invalidation
    of the caches) that a default event performs, which HIP documents as the
    way to time GPU work precisely on AMD devices.  A default event pair
    around one split launch read 3-4% (about 8 us) more than the kernel's
    own duration in a kernel trace.  Times are read after a device
    synchronization, so nothing relies on the fence.  Used like torch's
    timing events: record(stream), then start.elapsed_time(end) in ms."""
    FLAGS = 0x20000000  # hipEventDisableSystemFence
    _hip = None

    @classmethod
    def _lib(cls):
        if cls._hip is None:
            import ctypes
            torch.cuda.init()
            # the HIP runtime this process already uses (torch's), so that its
            # stream handles are valid here
            paths = sorted({ln.split()[-1] for ln in open("/proc/self/maps") if "libamdhip64" in ln})
            if not paths:
                raise RuntimeError("no HIP runtime loaded")
            h = ctypes.CDLL(paths[0])
            h.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            h.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
            h.hipEventDestroy.argtypes = [ctypes.c_void_p]
            cls._hip = (h, ctypes)
        return cls._hip

    def __init__(self):
        h, ct = self._lib()
        self.ev = ct.c_void_p()
        if h.hipEventCreateWithFlags(ct.byref(self.ev), self.FLAGS) != 0:
            raise RuntimeError("hipEventCreateWithFlags failed")

    def record(self, stream):
        h, ct = self._lib()
        if h.hipEventRecord(self.ev, ct.c_void_p(stream.cuda_stream)) != 0:
            raise RuntimeError("hipEventRecord failed")

    def elapsed_time(self, end):
        h, ct = self._lib()
        ms = ct.c_float()
        if h.hipEventElapsedTime(ct.byref(ms), self.ev, end.ev) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(ms.value)

    def __del__(self):
        if self._hip is not None and self.ev:
            self._hip[0].hipEventDestroy(self.ev)

WORKLOADS = {
    "batched": dict(config=2, formats=["INT8_G64", "FP8_ROW", "FP8_TENSOR"],
                    label="batched decode: 32 sequences x U[8192,32768] cached tokens, 24 q / 4 kv heads, "
                          "head_dim 256, 64-token pages"),
    "long": dict(config=3, formats=["NVFP4_G16", "NVFP4_G16/2L", "MXFP4"],
                 label="long-context decode: 1 sequence x 262144 tokens, 24 q / 4 kv heads, head_dim 256"),
    "long8": dict(config="3b", formats=["NVFP4_G16"],
                  label="long-context decode: 8 sequences x 65536 tokens, 24 q / 4 kv heads, head_dim 256"),
    "mixed": dict(config=4, formats=["K8V4"],
                  label="mixed-length decode: 64 sequences x logU[1K,128K] tokens, 24 q / 4 kv heads, head_dim 256"),
    "mtp": dict(config=5, formats=["MXFP8", "MXFP8/QMX"],
                label="MTP decode: 256 sequences x 4096 tokens, 4 query tokens, MHA 32 heads, head_dim 128, "
                      "128-token pages"),
    "tiny": dict(config=1, formats=["BF16", "FP8_ROW"],
                 label="tiny decode: 1 sequence x 1024 tokens, 4 q / 2 kv heads, head_dim 256"),
}

def parse_label(label):
    """'NVFP4_G16/2L' -> ('NVFP4_G16', True, False): a format, whether its
    NVFP4 planes take a calibrated per-tensor (second-level) scale, and
    ('MXFP8/QMX') whether decode runs in the query-MXFP8 mode."""
    fmt, _, mod = label.partition("/")
    return fmt, mod == "2L", mod == "QMX"


# formats whose split kernel has a packed variant for at most 8 query rows
# per kv head (G * n_q), by head_dim; the library picks it by itself
PACKED_SPLIT = {"INT8_G64": 256, "NVFP4_G16": 256, "MXFP4": 256}
PACK_MAX_ROWS = 8
VARIANT_QMX, VARIANT_PACK = 0x100, 0x200
# formats whose chunked prefill runs on the 32-row kernel (K exact in bf16,
# one query piece); the others keep the 16-row kernel
WIDE_PREFILL = ("BF16", "FP8_ROW", "FP8_TENSOR", "MXFP8", "K8V4")


def split_kernel_name(label, D, rows, fused=False):
    """The decode_split_kernel instantiation the library launches for one
    workload: the format id with its variant bits, the head dim, and
    whether the step's append is fused in."""
    fmt, _, qmx = parse_label(label)
    v = kvq.FORMATS[fmt]
    if qmx:
        v |= VARIANT_QMX
    elif PACKED_SPLIT.get(fmt) == D and rows <= PACK_MAX_ROWS:
        v |= VARIANT_PACK
    return "decode_split_kernel<%d, %d, %s>" % (v, D, "true" if fused else "false")


def kv_bytes_per_token(d):
    return kvq.page_bytes(d) // (d.page_size * d.num_kv_heads)


class Setup:
    """One workload resident on the GPU: pool, tables, and the step's inputs."""

    def __init__(self, config, label):
        fmt, two_level, qmx = parse_label(label)
        self.flags = kvq.SPLIT_WRITE_WHOLE_UNITS | (kvq.SPLIT_Q_MXFP8 if qmx else 0)
        self.case = c = W.make_case(config, fmt, device="cuda", two_level=two_level)
        self.desc = kvq.desc(c.fmt, c.D, c.P, c.H_kv, c.num_pages, c.k_scale, c.v_scale)
        self.pool = kvq.alloc_pool(self.desc)
        kvq.quantize_append(self.desc, self.pool, c.k, c.v, c.slot_mapping)  # fill the cache
        self.bt = torch.as_tensor(c.block_table, device="cuda")
        self.sl = torch.as_tensor(c.seq_lens, device="cuda")
        # the step appends each sequence's n_q newest tokens (positions
        # L_b - n_q .. L_b - 1, the decoded or drafted ones) again
        lens = c.seq_lens.astype(np.int64)
        idx = (np.cumsum(lens) - c.n_q)[:, None] + np.arange(c.n_q)[None, :]
        idx = torch.as_tensor(idx.reshape(-1), device="cuda")
        self.k_new = c.k.index_select(0, idx).view(c.B, c.n_q, c.H_kv, c.D).contiguous()
        self.v_new = c.v.index_select(0, idx).view(c.B, c.n_q, c.H_kv, c.D).contiguous()
        self.slot_new = c.slot_mapping.index_select(0, idx).contiguous()
        self.q = c.q
        self.nwg, self.slots = kvq.decode_plan(self.desc, c.B, c.n_q, c.H_q, c.max_pages)
        self.ws = kvq.alloc_workspace(kvq.workspace_size(self.desc, c.B, c.n_q, c.H_q, c.max_pages))
        self.out = torch.empty((c.B, c.n_q, c.H_q, c.D), dtype=torch.float32, device="cuda")
        self.lse = torch.empty((c.B, c.n_q, c.H_q), dtype=torch.float32, device="cuda")
        self.bpt = kv_bytes_per_token(self.desc)
        self.kv_bytes = int(c.seq_lens.astype(np.int64).sum()) * c.H_kv * self.bpt
        torch.cuda.synchronize()

    def step(self, stream, ev=None, fused=True, phases=False):
        """One decode step: append the new tokens, attend, reduce.  Fused: the
        two launches kvq_decode_step makes (the split kernel stores the new
        tokens); else quantize-append and the two launches of
        kvq_decode_attention.  Events: ev[0] before and ev[3] after the step,
        and with phases=True also ev[1], ev[2] between its launches (each
        recorded event costs the stream a few microseconds, so a step is
        timed without them and its phases in a series of their own)."""
        c = self.case
        rec = (lambda i: ev[i].record(stream)) if ev is not None else (lambda i: None)
        inner = rec if phases else (lambda i: None)
        rec(0)
        if fused:
            kvq.decode_step_split(self.desc, self.pool, self.k_new, self.v_new, self.q, self.bt, self.sl,
                                  c.softmax_scale, self.ws, flags=self.flags, out=self.out,
                                  lse=self.lse, stream=stream)
        else:
            kvq.quantize_append(self.desc, self.pool, self.k_new.view(-1, c.H_kv, c.D),
                                self.v_new.view(-1, c.H_kv, c.D), self.slot_new, stream=stream)
            inner(1)
            kvq.decode_split(self.desc, self.pool, self.q, self.bt, self.sl, c.softmax_scale, self.ws,
                             flags=self.flags, out=self.out, lse=self.lse, stream=stream)
        inner(2)
        kvq.decode_combine(self.desc, c.B, c.n_q, c.H_q, c.max_pages, self.sl, self.ws, self.out, self.lse,
                           flags=self.flags, stream=stream)
        rec(3)


class Probe:
    """The streaming kernels of libkvq_probe.so; a 1 GiB buffer to flush with."""

    def __init__(self):
        from decode_attention_quant_amd import probe
        self.p = probe
        probe.library()
        self.buf = torch.ones(FLUSH_BYTES, dtype=torch.uint8, device="cuda")
        self.sink = torch.zeros(4, dtype=torch.int32, device="cuda")

    def flush(self, stream):
        self.p.read(self.buf, self.sink, stream)

    def rates(self, stream, reps=10):
        """Median GB/s of the read scan over 4 GiB with plain loads and with
        the non-temporal hint (the decode copies carry it), and of a 2 GiB
        copy (read + write counted), on a buffer freed afterwards."""
        buf = torch.ones(RATE_BYTES, dtype=torch.uint8, device="cuda")
        rd, nt, cp = [], [], []
        with torch.cuda.stream(stream):
            for i in range(reps + 2):
                e = [HipEvent() for _ in range(4)]
                e[0].record(stream)
                self.p.read(buf, self.sink, stream)
                e[1].record(stream)
                self.p.read(buf, self.sink, stream, nontemporal=True)
                e[2].record(stream)
                self.p.copy(buf[COPY_BYTES:], buf[:COPY_BYTES], stream)
                e[3].record(stream)
                torch.cuda.synchronize()
                if i >= 2:
                    rd.append(RATE_BYTES / (e[0].elapsed_time(e[1]) * 1e-3) / 1e9)
                    nt.append(RATE_BYTES / (e[1].elapsed_time(e[2]) * 1e-3) / 1e9)
                    cp.append(2 * COPY_BYTES / (e[2].elapsed_time(e[3]) * 1e-3) / 1e9)
        del buf
        torch.cuda.empty_cache()
        return float(np.median(rd)), float(np.median(nt)), float(np.median(cp))


def _stats(x):
    return {"mean": float(np.mean(x)), "median": float(np.median(x)), "p10": float(np.percentile(x, 10)),
            "p90": float(np.percentile(x, 90))}


def time_steps(s, steps, warmup, stream, probe=None, fused=True, phases=False):
    """Per-step HIP-event times (ms) of the step (events at its ends only),
    or with phases=True of its launches (events between them too).

    With a probe, its cache-evicting read runs before each step, outside
    the step's events; the wall time between the first and last step then
    includes those reads."""
    # no garbage collection while steps are being launched: a collector pause
    # between the launches of one step would show up as GPU idle time inside
    # its events (seen as single steps of tens of ms)
    gc.collect()
    gc.disable()
    try:
        return _time_steps(s, steps, warmup, stream, probe, fused, phases)
    finally:
        gc.enable()


def _time_steps(s, steps, warmup, stream, probe, fused, phases):
    with torch.cuda.stream(stream):
        for _ in range(warmup):
            if probe is not None:
                probe.flush(stream)
            s.step(stream, fused=fused)
        torch.cuda.synchronize()
        t0 = HipEvent()
        t1 = HipEvent()
        evs = [[HipEvent() for _ in range(4)] for _ in range(steps)]
        t0.record(stream)
        for i in range(steps):
            if probe is not None:
                probe.flush(stream)
            s.step(stream, evs[i], fused=fused, phases=phases)
        t1.record(stream)
        torch.cuda.synchronize()
    t = {"wall": t0.elapsed_time(t1) / steps, "step": _stats([e[0].elapsed_time(e[3]) for e in evs])}
    if phases:
        t["combine"] = _stats([e[2].elapsed_time(e[3]) for e in evs])
        if fused:
            t["split"] = _stats([e[0].elapsed_time(e[2]) for e in evs])
        else:
            t["append"] = _stats([e[0].elapsed_time(e[1]) for e in evs])
            t["split"] = _stats([e[1].elapsed_time(e[2]) for e in evs])
    return t


def append_chunk_bench(formats, stream, probe, reps=10):
    """Quantize-append of one 2048-token chunk per sequence of the mixed-length
    workload (64 sequences, chunks starting mid-page): tok/s and GB/s moved,
    against the HBM roof T * H_kv * (4 D + bytes_per_token) / 8 TB/s."""
    res = {}
    for label in formats:
        fmt, two_level, _ = parse_label(label)
        c = W.make_case(4, fmt, device="cuda", reserve=APPEND_CHUNK, two_level=two_level)
        c.k = c.v = None  # only the new chunk is written
        d = kvq.desc(c.fmt, c.D, c.P, c.H_kv, c.num_pages, 1.0, 1.0)
        if fmt == "FP8_TENSOR" or two_level:  # the cached tensors' calibrated scales
            d = kvq.desc(c.fmt, c.D, c.P, c.H_kv, c.num_pages, c.k_scale, c.v_scale)
        pool = kvq.alloc_pool(d)
        k, v, slots = W.append_chunk(c, APPEND_CHUNK, device="cuda")
        T = k.shape[0]
        bpt = kv_bytes_per_token(d)
        moved = T * c.H_kv * (4 * c.D + bpt)
        ts = []
        with torch.cuda.stream(stream):
            for i in range(reps + 2):
                probe.flush(stream)
                e = [HipEvent() for _ in range(2)]
                e[0].record(stream)
                kvq.quantize_append(d, pool, k, v, slots, stream=stream)
                e[1].record(stream)
                if i >= 2:
                    ts.append(e)
            torch.cuda.synchronize()
        ms = float(np.median([e[0].elapsed_time(e[1]) for e in ts]))
        roof = HBM_PEAK_GBS * 1e9 / (c.H_kv * (4 * c.D + bpt))
        res[label] = {"tokens": T, "ms": ms, "tok_per_s": T / (ms * 1e-3), "GB_per_s": moved / (ms * 1e-3) / 1e9,
                    "roof_tok_per_s": roof, "frac_of_roof": T / (ms * 1e-3) / roof}
        print("[bench] append %s: %d tokens in %.3f ms, %.1f M tok/s (%.1f%% of the HBM roof), %.0f GB/s" % (
            label, T, ms, T / ms / 1e3, 100 * res[label]["frac_of_roof"], res[label]["GB_per_s"]),
            file=sys.stderr, flush=True)
        del pool, k, v, slots, c
        torch.cuda.empty_cache()
    return res


def prefill_bench(stream, probe, chunk=APPEND_CHUNK, fmt="K8V4", reps=3):
    """Chunked prefill of the mixed-length workload: 64 sequences of
    ~U(ln 1K, ln 128K) cached tokens, each followed by a `chunk`-token prefill
    chunk (appended through the write path, untimed); then every chunk query
    attends causally over its sequence's cache (timed).  Attention flops are
    4 D H_q per visible (query, position) pair; the kernel's matrix products
    are f16/bf16, so the roof is the 2.5 PFLOP/s dense peak."""
    c = W.make_case(4, fmt, device="cuda", n_q=chunk, reserve=chunk)
    d = kvq.desc(c.fmt, c.D, c.P, c.H_kv, c.num_pages, c.k_scale, c.v_scale)
    pool = kvq.alloc_pool(d)
    kvq.quantize_append(d, pool, c.k, c.v, c.slot_mapping)
    k, v, slots = W.append_chunk(c, chunk, device="cuda")
    kvq.quantize_append(d, pool, k, v, slots)
    del k, v, slots
    c.k = c.v = None
    torch.cuda.empty_cache()
    lens = c.seq_lens.astype(np.int64)
    sl = torch.as_tensor((lens + chunk).astype(np.int32), device="cuda")
    bt = torch.as_tensor(c.block_table, device="cuda")
    out = torch.empty(c.q.shape, dtype=torch.float32, device="cuda")
    visible = int(np.sum(chunk * (lens + 1) + chunk * (chunk - 1) // 2))  # sum over queries of positions seen
    flops = 4.0 * c.D * c.H_q * visible
    ts = []
    with torch.cuda.stream(stream):
        for i in range(reps + 1):
            probe.flush(stream)
            e = [HipEvent() for _ in range(2)]
            e[0].record(stream)
            kvq.prefill_attention(d, pool, c.q, bt, sl, c.softmax_scale, out=out, stream=stream)
            e[1].record(stream)
            if i >= 1:
                ts.append(e)
        torch.cuda.synchronize()
    ms = [e[0].elapsed_time(e[1]) for e in ts]
    mean = float(np.mean(ms))
    tflops = flops / (mean * 1e-3) / 1e12
    kv_bytes = int((lens + chunk).sum()) * c.H_kv * kv_bytes_per_token(d)
    res = {"workload": "64 sequences x one %d-token prefill chunk after U(ln 1K, ln 128K) cached tokens, "
                       "24 q / 4 kv heads, head_dim 256, causal over the cache" % chunk,
           "kv_dtype": fmt, "query_tokens": int(c.B * chunk), "attention_flops": flops,
           "ms": mean, "ms_runs": ms, "TFLOP_per_s": tflops,
           "roofline": {"bound": "mfma", "achieved": tflops, "peak": MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                        "frac": tflops / MFMA_PEAK_TFLOPS, "kernel": "%s<%d, %d> (%s)" % (
                            "prefill_wide_kernel" if fmt in WIDE_PREFILL else "prefill_kernel", kvq.FORMATS[fmt],
                            c.D, fmt)},
           "kv_bytes_per_call": kv_bytes, "row_tiles": int(c.B * c.H_kv * ((6 * chunk + 63) // 64))}
    print("[bench] prefill %s: %d query tokens over %.2f GB of cache in %.2f ms, %.0f TFLOP/s (%.1f%% of %.0f)" % (
        fmt, c.B * chunk, kv_bytes / 1e9, mean, tflops, 100 * tflops / MFMA_PEAK_TFLOPS, MFMA_PEAK_TFLOPS),
        file=sys.stderr, flush=True)
    del pool, out, c
    torch.cuda.empty_cache()
    return res


# the sources the split kernel is compiled from, and the planner that sizes
# its grid (the partials' bytes depend on the workgroup count)
SPLIT_SOURCES = ["kvq_decode.hip", "kvq_decode_core.hpp", "kvq_device.hpp", "kvq_encode.hpp", "kvq_format.hpp",
                 "kvq_internal.hpp", "kvq_api.hip"]


def _code_only(text):
    """C++ source without its comments and blank lines: an edit of the prose
    alone leaves the recorded counters valid."""
    import re
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return "\n".join(ln.rstrip() for ln in text.splitlines() if ln.strip())


def kernel_sources_sha():
    """SHA-256 of the split kernel's sources (code only, comments dropped)."""
    h = hashlib.sha256()
    for f in SPLIT_SOURCES:
        h.update(f.encode())
        with open(os.path.join(CSRC, f), encoding="utf-8") as fh:
            h.update(_code_only(fh.read()).encode())
    return h.hexdigest()


def recorded_traffic(workload, fmt):
    """HBM bytes per split-kernel launch from the committed counter
    summaries, or None when none covers this workload and format or the
    split kernel's sources changed since they were taken."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    with open(TRAFFIC_FILE) as fh:
        records = json.load(fh)
    sha = kernel_sources_sha()
    for t in records if isinstance(records, list) else [records]:
        if t.get("sources_sha256") == sha and t.get("workload") == workload and t.get("kv_dtype") == fmt:
            return t["traffic_bytes_per_launch"]
    return None


def _counter_means(folder, counter):
    """Mean per-dispatch value of ``counter`` by kernel name, from rocprofv3 CSVs."""
    vals = {}
    files = glob.glob(os.path.join(folder, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit("no counter_collection.csv under %s" % folder)
    for f in files:
        with open(f) as fh:
            for row in csv.DictReader(fh):
                if row.get("Counter_Name") != counter:
                    continue
                key = (row["Kernel_Name"], row.get("Dispatch_Id", len(vals)))
                vals[key] = vals.get(key, 0.0) + float(row["Counter_Value"])
    by_kernel = {}
    for (name, _), v in vals.items():
        by_kernel.setdefault(name, []).append(v)
    return {k: (float(np.mean(v)), len(v)) for k, v in by_kernel.items()}


def summarize_counters(fetch_dir, write_dir, bench_json):
    with open(bench_json) as fh:
        line = json.loads([ln for ln in fh if ln.startswith("{")][-1])
    fmt = line["config"]["kv_dtype"]
    fetch = _counter_means(fetch_dir, "FETCH_SIZE")
    write = _counter_means(write_dir, "WRITE_SIZE")

    def pick(table, needle):
        hits = [(k, v) for k, v in table.items() if needle in k]
        if len(hits) != 1:
            raise SystemExit("expected one kernel matching %r, found %s" % (needle, [k for k, _ in hits]))
        return hits[0]

    cfg = line["config"]
    split_name = split_kernel_name(fmt, cfg["head_dim"], cfg["num_q_heads"] // cfg["num_kv_heads"] * cfg["n_q"])
    kname, (f_kib, n_f) = pick(fetch, split_name)
    _, (w_kib, n_w) = pick(write, split_name)
    _, (cf_kib, _) = pick(fetch, "kvq_probe::copy_kernel")
    _, (cw_kib, _) = pick(write, "kvq_probe::copy_kernel")
    copy_bytes = COPY_BYTES
    rf, wf = copy_bytes / 1024.0 / cf_kib, copy_bytes / 1024.0 / cw_kib
    traffic = (f_kib * rf + w_kib * wf) * 1024.0
    kv = line["per_kv_dtype"][fmt]["kv_bytes"]
    return {
        "kernel": kname, "workload": line["config"]["workload_name"], "kv_dtype": fmt,
        "sources_sha256": kernel_sources_sha(),
        "split_dispatches": [n_f, n_w],
        "fetch_kib_per_dispatch": f_kib, "write_kib_per_dispatch": w_kib,
        "copy_kernel_bytes_each_way": copy_bytes, "copy_fetch_kib": cf_kib, "copy_write_kib": cw_kib,
        "read_scale": rf, "write_scale": wf,
        "traffic_bytes_per_launch": traffic,
        "algorithmic_kv_bytes_per_launch": kv,
        "traffic_over_algorithmic": traffic / kv,
    }


def host_cpu_model():
    """The host CPU's model name from /proc/cpuinfo (None where it is absent)."""
    try:
        with open("/proc/cpuinfo") as fh:
            for ln in fh:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(s, budget_s=10.0):
    """The oracle as it stands, on whole sequences of the same workload (all
    kv heads; its pool built untimed), timed per decode step: append the
    n_q newest tokens, then fp64 attention over every cached page."""
    from threadpoolctl import threadpool_info
    from oracle import attention as OA, layout as OL

    c = s.case
    geo = OL.Geometry(c.fmt, c.D, c.P, c.H_kv)
    pool = np.full(c.num_pages * geo.page_bytes, 0xFF, dtype=np.uint8)
    q_bits = W.bf16_bits(c.q)
    elapsed, nbytes, seqs, tokens = 0.0, 0, 0, 0
    starts = np.concatenate([[0], np.cumsum(c.seq_lens.astype(np.int64))])
    for b in range(c.B):
        lo, hi = int(starts[b]), int(starts[b + 1])
        kb, vb = W.bf16_bits(c.k[lo:hi]), W.bf16_bits(c.v[lo:hi])
        slots = c.slot_mapping[lo:hi].cpu().numpy()
        n = c.n_q
        OA.quantize_append(geo, pool, kb[:-n], vb[:-n], slots[:-n], c.k_scale, c.v_scale)  # resident cache
        t = time.perf_counter()
        OA.quantize_append(geo, pool, kb[-n:], vb[-n:], slots[-n:], c.k_scale, c.v_scale)  # the step's append
        OA.attention_ref(geo, pool, q_bits, c.block_table, c.seq_lens, c.softmax_scale, c.n_q, c.k_scale,
                         c.v_scale, only=[(b, h) for h in range(c.H_kv)])
        elapsed += time.perf_counter() - t
        nbytes += (hi - lo) * c.H_kv * s.bpt
        seqs += 1
        tokens += hi - lo
        if elapsed >= budget_s:
            break
    blas = [i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"]
    return {"value": nbytes / elapsed / 1e9, "unit": "GB/s", "cores": int(max(blas) if blas else 1),
            "kind": "oracle", "host_cpu": host_cpu_model(), "host_logical_cpus": os.cpu_count(),
            "sample": "%d whole sequences (%d cached tokens x %d kv heads) of the same workload; one step each: "
                      "append the n_q newest tokens, then fp64 attention over all cached pages; %.1f s" % (
                          seqs, tokens, c.H_kv, elapsed)}


def run_workload(name, formats, args, stream, flush):
    """Time the step of every format of one workload.  Returns (per-format
    records, the first format's Setup kept resident for the caller)."""
    wl = WORKLOADS[name]
    per = {}
    primary = None
    for fmt in formats:
        print("[bench] %s %s: building the cache" % (name, fmt), file=sys.stderr, flush=True)
        s = Setup(wl["config"], fmt)
        # the step as append + decode (the headline), then as one fused step,
        # after a few untimed steps of each (the first steps after the cache
        # is built run slower)
        for fused in (False, True):
            time_steps(s, 3, 1, stream, flush, fused=fused)
        t = time_steps(s, args.steps, args.warmup, stream, flush, fused=False)
        tf = time_steps(s, args.steps, args.warmup, stream, flush, fused=True)
        # the launches of each step apart (events between them), for the
        # split kernel's own time and the breakdown
        tp = time_steps(s, args.steps, args.warmup, stream, flush, fused=False, phases=True)
        tpf = time_steps(s, args.steps, args.warmup, stream, flush, fused=True, phases=True)
        ms = t["step"]["mean"] if flush is not None else t["wall"]
        ms_f = tf["step"]["mean"] if flush is not None else tf["wall"]
        c = s.case
        split_ms = tp["split"]["mean"]
        achieved = s.kv_bytes / (split_ms * 1e-3) / 1e9
        fmt_base = parse_label(fmt)[0]
        res = {
            "GB_per_s": s.kv_bytes / (ms * 1e-3) / 1e9,
            "pct_of_hbm_peak": 100.0 * s.kv_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "ms_per_step": ms,
            "step_us": 1000.0 * ms,
            "step_ms": t["step"], "wall_ms_per_step": t["wall"],
            "kv_bytes": s.kv_bytes,
            "bytes_per_token": s.bpt,
            "new_tokens_per_step": c.B * c.n_q,
            "split_kernel_ms": tp["split"], "combine_ms": tp["combine"], "step_append_ms": tp["append"],
            "phase_times_note": "split_kernel_ms, combine_ms and step_append_ms come from a series with events "
                                "between the launches; the step times have events at their ends only",
            "split_workgroups": s.nwg, "partial_slots": s.slots,
            "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": achieved / HBM_PEAK_GBS,
                         "kernel": "%s (%s)" % (split_kernel_name(fmt, c.D, c.H_q // c.H_kv * c.n_q), fmt),
                         "kernel_ms": split_ms, "algorithmic_bytes_per_launch": s.kv_bytes,
                         "traffic": recorded_traffic(name, fmt)},
            "fused_step": {
                "GB_per_s": s.kv_bytes / (ms_f * 1e-3) / 1e9,
                "pct_of_hbm_peak": 100.0 * s.kv_bytes / (ms_f * 1e-3) / 1e9 / HBM_PEAK_GBS,
                "ms_per_step": ms_f, "step_ms": tf["step"],
                "split_kernel_ms": tpf["split"], "combine_ms": tpf["combine"]},
        }
        per[fmt] = res
        print("[bench] %s %s: %.1f GB/s (%.1f%% of peak), step %.3f ms (launches apart: append %.3f, split %.3f "
              "(p10 %.3f p90 %.3f, %.1f%% of peak), combine %.3f) | fused step %.1f GB/s: %.3f ms (apart: split "
              "storing the new tokens %.3f, combine %.3f)" % (
                  name, fmt, res["GB_per_s"], res["pct_of_hbm_peak"], ms, tp["append"]["mean"],
                  split_ms, tp["split"]["p10"], tp["split"]["p90"], 100 * achieved / HBM_PEAK_GBS,
                  tp["combine"]["mean"], res["fused_step"]["GB_per_s"], ms_f, tpf["split"]["mean"],
                  tpf["combine"]["mean"]),
              file=sys.stderr, flush=True)
        if primary is None:
            primary = s
        else:
            del s
            torch.cuda.empty_cache()
    return per, primary


HEADLINE = "batched"  # the batched decode workload is the one the metric is quoted on


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="all", choices=["all"] + sorted(WORKLOADS),
                    help="'all' (the default) times every workload and reports the batched one as the headline")
    ap.add_argument("--formats", default=None, help="comma-separated subset of a single workload's formats")
    ap.add_argument("--append-formats", default=",".join(APPEND_FORMATS),
                    help="formats of the prefill-chunk append measurement, or 'none'")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true", help="skip the chunked-prefill attention measurement")
    ap.add_argument("--prefill-formats", default="K8V4",
                    help="comma-separated formats of the chunked-prefill measurement (the first is the headline)")
    ap.add_argument("--no-flush", action="store_true", help="time steps back to back, caches warm")
    ap.add_argument("--cpu-budget", type=float, default=10.0)
    ap.add_argument("--summarize-counters", nargs="+", metavar="DIR_OR_JSON",
                    help="FETCH_DIR WRITE_DIR BENCH_JSON triples")
    args = ap.parse_args()
    if args.summarize_counters:
        a = args.summarize_counters
        if len(a) % 3:
            ap.error("--summarize-counters takes FETCH_DIR WRITE_DIR BENCH_JSON triples")
        print(json.dumps([summarize_counters(*a[i:i + 3]) for i in range(0, len(a), 3)], indent=1))
        return
    if args.gpus != 1:
        print("bench.py measures one GPU: this build runs the hot path on a single device and has no "
              "multi-GPU mode; run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    if args.formats and args.workload == "all":
        print("--formats needs a single --workload", file=sys.stderr)
        sys.exit(2)
    kvq.library()
    head = HEADLINE if args.workload == "all" else args.workload
    names = [head] + [n for n in WORKLOADS if n != head] if args.workload == "all" else [head]
    stream = torch.cuda.Stream()
    probe = Probe()
    plain_gbs, read_gbs, copy_gbs = probe.rates(stream)
    print("[bench] streaming read %.0f GB/s (non-temporal loads; %.0f plain), copy %.0f GB/s (read + write)" % (
        read_gbs, plain_gbs, copy_gbs), file=sys.stderr, flush=True)
    flush = None if args.no_flush else probe
    per_workload = {}
    primary = None
    for name in names:
        formats = args.formats.split(",") if args.formats else WORKLOADS[name]["formats"]
        per, s = run_workload(name, formats, args, stream, flush)
        per_workload[name] = {"workload": WORKLOADS[name]["label"], "per_kv_dtype": per}
        if name == head:
            primary = (formats[0], s, per[formats[0]], per)
        else:
            del s
            torch.cuda.empty_cache()
    fmt, s, res, per = primary
    c = s.case
    split_ms = res["split_kernel_ms"]["mean"]
    achieved = s.kv_bytes / (split_ms * 1e-3) / 1e9
    append_formats = [] if args.append_formats == "none" else args.append_formats.split(",")
    appends = append_chunk_bench(append_formats, stream, probe) if append_formats else {}
    prefill = None
    if not args.no_prefill:
        pf_formats = [f for f in args.prefill_formats.split(",") if f]
        runs = {f: prefill_bench(stream, probe, fmt=f) for f in pf_formats}
        prefill = dict(runs[pf_formats[0]])
        if len(pf_formats) > 1:
            prefill["per_kv_dtype"] = runs
    line = {
        "metric": METRIC,
        "value": res["GB_per_s"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": res["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": WORKLOADS[head]["label"], "workload_name": head, "kv_dtype": fmt, "batch": c.B,
                   "n_q": c.n_q, "num_q_heads": c.H_q, "num_kv_heads": c.H_kv, "head_dim": c.D,
                   "page_size": c.P, "cached_tokens": int(c.seq_lens.astype(np.int64).sum()),
                   "split_workgroups": s.nwg, "cache_flush_between_steps": flush is not None},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": recorded_traffic(head, fmt),
                     "kernel": "%s (%s)" % (split_kernel_name(fmt, c.D, c.H_q // c.H_kv * c.n_q), fmt),
                     "kernel_ms": split_ms,
                     "algorithmic_bytes_per_launch": s.kv_bytes,
                     "measured_streaming_read_GBs": read_gbs, "frac_of_measured_read": achieved / read_gbs,
                     "measured_plain_load_read_GBs": plain_gbs, "measured_copy_GBs": copy_gbs},
        "pct_of_hbm_peak": res["pct_of_hbm_peak"],
        "quant_append": ({"workload": "64 sequences x one %d-token prefill chunk (mixed lengths 1K-128K, "
                                      "chunks start mid-page), 4 kv heads, head_dim 256" % APPEND_CHUNK,
                          "kv_dtype": append_formats[0], **appends[append_formats[0]],
                          "per_kv_dtype": appends} if appends else None),
        "per_kv_dtype": per,
        "per_workload": per_workload,
        "prefill_attention": prefill,
    }
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle) on %s" % fmt, file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(s, args.cpu_budget)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
