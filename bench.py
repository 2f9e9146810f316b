"""Benchmark: one decode step of the quantized paged-KV hot path on MI355X.

A step is the whole hot path over one batch: quantize-append of each
sequence's newest token (K and V of every kv head, through the codec and the
Hadamard rotation where the format has it), then split-K decode attention
over every cached page and the cross-split combine.  Inputs are resident in
HBM before timing starts.  The default workload is the batched decode:
32 sequences with contexts drawn uniformly from 8K-32K tokens, 24 query /
4 KV heads, head_dim 256, 64-token pages, for each of INT8-G64, FP8 row-256
and per-tensor FP8 (the headline value is INT8-G64).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload batched]

Prints one JSON line.  ``value`` is effective compressed-KV bandwidth:
sum_b H_kv * L_b * bytes_per_token / ms_per_step.  ``roofline`` prices the
dominant kernel (the split kernel) against the 8 TB/s HBM peak with its
average duration measured by HIP events on its own stream; ``cpu_baseline``
times the CPU oracle on a bounded sample of the same workload.
"""

import argparse
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
METRIC = "decode-attn effective KV GB/s (% of HBM peak) per kv-dtype; quant-append tok/s"

WORKLOADS = {
    "batched": dict(config=2, formats=["INT8_G64", "FP8_ROW", "FP8_TENSOR"],
                    label="batched decode: 32 sequences x U[8192,32768] cached tokens, 24 q / 4 kv heads, "
                          "head_dim 256, 64-token pages"),
    "long": dict(config=3, formats=["NVFP4_G16"],
                 label="long-context decode: 1 sequence x 262144 tokens, 24 q / 4 kv heads, head_dim 256"),
    "long8": dict(config="3b", formats=["NVFP4_G16"],
                  label="long-context decode: 8 sequences x 65536 tokens, 24 q / 4 kv heads, head_dim 256"),
    "mixed": dict(config=4, formats=["K8V4"],
                  label="mixed-length decode: 64 sequences x logU[1K,128K] tokens, 24 q / 4 kv heads, head_dim 256"),
    "mtp": dict(config=5, formats=["MXFP8"],
                label="MTP decode: 256 sequences x 4096 tokens, 4 query tokens, MHA 32 heads, head_dim 128, "
                      "128-token pages"),
    "tiny": dict(config=1, formats=["BF16", "FP8_ROW"],
                 label="tiny decode: 1 sequence x 1024 tokens, 4 q / 2 kv heads, head_dim 256"),
}

def kv_bytes_per_token(d):
    return kvq.page_bytes(d) // (d.page_size * d.num_kv_heads)


class Setup:
    """One workload resident on the GPU: pool, tables, and the step's inputs."""

    def __init__(self, config, fmt):
        self.case = c = W.make_case(config, fmt, device="cuda")
        self.desc = kvq.desc(c.fmt, c.D, c.P, c.H_kv, c.num_pages, c.k_scale, c.v_scale)
        self.pool = kvq.alloc_pool(self.desc)
        kvq.quantize_append(self.desc, self.pool, c.k, c.v, c.slot_mapping)  # fill the cache
        self.bt = torch.as_tensor(c.block_table, device="cuda")
        self.sl = torch.as_tensor(c.seq_lens, device="cuda")
        # the step appends each sequence's newest token (position L_b - 1) again
        last = np.cumsum(c.seq_lens.astype(np.int64)) - 1
        idx = torch.as_tensor(last, device="cuda")
        self.k_new = c.k.index_select(0, idx).contiguous()
        self.v_new = c.v.index_select(0, idx).contiguous()
        self.slot_new = c.slot_mapping.index_select(0, idx).contiguous()
        self.q = c.q
        self.nwg, self.slots = kvq.decode_plan(self.desc, c.B, c.n_q, c.H_q, c.max_pages)
        self.ws = kvq.alloc_workspace(kvq.workspace_size(self.desc, c.B, c.n_q, c.H_q, c.max_pages))
        self.out = torch.empty((c.B, c.n_q, c.H_q, c.D), dtype=torch.float32, device="cuda")
        self.lse = torch.empty((c.B, c.n_q, c.H_q), dtype=torch.float32, device="cuda")
        self.bpt = kv_bytes_per_token(self.desc)
        self.kv_bytes = int(c.seq_lens.astype(np.int64).sum()) * c.H_kv * self.bpt
        torch.cuda.synchronize()

    def step(self, stream, ev=None):
        c = self.case
        if ev is not None:
            ev[0].record(stream)
        kvq.quantize_append(self.desc, self.pool, self.k_new, self.v_new, self.slot_new, stream=stream)
        if ev is not None:
            ev[1].record(stream)
        # the two launches kvq_decode_attention makes, timed apart
        kvq.decode_split(self.desc, self.pool, self.q, self.bt, self.sl, c.softmax_scale, self.ws,
                         flags=kvq.SPLIT_WRITE_WHOLE_UNITS, out=self.out, lse=self.lse, stream=stream)
        if ev is not None:
            ev[2].record(stream)
        kvq.decode_combine(self.desc, c.B, c.n_q, c.H_q, c.max_pages, self.sl, self.ws, self.out, self.lse,
                           flags=kvq.SPLIT_WRITE_WHOLE_UNITS, stream=stream)
        if ev is not None:
            ev[3].record(stream)


def time_steps(s, steps, warmup, stream):
    with torch.cuda.stream(stream):
        for _ in range(warmup):
            s.step(stream)
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
        t0.record(stream)
        for i in range(steps):
            s.step(stream, evs[i])
        t1.record(stream)
        torch.cuda.synchronize()
        total = t0.elapsed_time(t1)
        app = [e[0].elapsed_time(e[1]) for e in evs]
        dec = [e[1].elapsed_time(e[2]) for e in evs]   # split kernel
        comb = [e[2].elapsed_time(e[3]) for e in evs]
    return total / steps, float(np.mean(app)), float(np.mean(dec)), float(np.mean(comb)), \
        float(np.percentile(dec, 10)), float(np.percentile(dec, 90))


def cpu_baseline(s, budget_s=10.0):
    """The oracle as it stands, on whole sequences of the same workload (all
    kv heads; its pool built untimed), timed per decode step: append the
    newest token, then fp64 attention over every cached page."""
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
        OA.quantize_append(geo, pool, kb[:-1], vb[:-1], slots[:-1], c.k_scale, c.v_scale)  # resident cache
        t = time.perf_counter()
        OA.quantize_append(geo, pool, kb[-1:], vb[-1:], slots[-1:], c.k_scale, c.v_scale)  # the step's append
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
            "kind": "oracle",
            "sample": "%d whole sequences (%d cached tokens x %d kv heads) of the same workload; one step each: "
                      "append the newest token, then fp64 attention over all cached pages; %.1f s" % (
                          seqs, tokens, c.H_kv, elapsed)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="batched", choices=sorted(WORKLOADS))
    ap.add_argument("--formats", default=None, help="comma-separated subset of the workload's formats")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=10.0)
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: this build runs the hot path on a single device and has no "
              "multi-GPU mode; run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    kvq.library()
    wl = WORKLOADS[args.workload]
    formats = args.formats.split(",") if args.formats else wl["formats"]
    stream = torch.cuda.Stream()
    per = {}
    primary = None
    for fmt in formats:
        print("[bench] %s %s: building the cache" % (args.workload, fmt), file=sys.stderr, flush=True)
        s = Setup(wl["config"], fmt)
        ms, app_ms, split_ms, comb_ms, p10, p90 = time_steps(s, args.steps, args.warmup, stream)
        c = s.case
        res = {
            "GB_per_s": s.kv_bytes / (ms * 1e-3) / 1e9,
            "pct_of_hbm_peak": 100.0 * s.kv_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "ms_per_step": ms,
            "kv_bytes": s.kv_bytes,
            "bytes_per_token": s.bpt,
            "split_kernel_ms": split_ms, "split_kernel_ms_p10": p10, "split_kernel_ms_p90": p90,
            "combine_ms": comb_ms,
            "append_ms": app_ms,
            "append_tok_per_s": c.B / (app_ms * 1e-3),
            "split_workgroups": s.nwg, "partial_slots": s.slots,
        }
        per[fmt] = res
        print("[bench] %s %s: %.1f GB/s (%.1f%% of peak), step %.3f ms, split %.3f ms, combine %.3f ms, "
              "append %.3f ms" % (args.workload, fmt, res["GB_per_s"], res["pct_of_hbm_peak"], ms, split_ms,
                                  comb_ms, app_ms), file=sys.stderr, flush=True)
        if primary is None:
            primary = (fmt, s, res)
        else:
            del s
            torch.cuda.empty_cache()
    fmt, s, res = primary
    c = s.case
    achieved = s.kv_bytes / (res["split_kernel_ms"] * 1e-3) / 1e9
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
        "config": {"workload": wl["label"], "kv_dtype": fmt, "batch": c.B, "n_q": c.n_q, "num_q_heads": c.H_q,
                   "num_kv_heads": c.H_kv, "head_dim": c.D, "page_size": c.P,
                   "cached_tokens": int(c.seq_lens.astype(np.int64).sum()),
                   "split_workgroups": s.nwg},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": None,
                     "kernel": "decode_split_kernel<%s>" % fmt, "kernel_ms": res["split_kernel_ms"]},
        "pct_of_hbm_peak": res["pct_of_hbm_peak"],
        "quant_append": {"tokens_per_step": c.B, "tok_per_s": res["append_tok_per_s"], "ms": res["append_ms"]},
        "per_kv_dtype": {k: {kk: (round(vv, 4) if isinstance(vv, float) else vv) for kk, vv in v.items()}
                         for k, v in per.items()},
    }
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle) on %s" % fmt, file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(s, args.cpu_budget)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
