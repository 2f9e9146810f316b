"""CPU oracle for the quantized paged-KV cache and its decode attention.

TEST INFRASTRUCTURE ONLY.  This package is a plain, slow, deliberately
unoptimised NumPy description of what the GPU library computes.  Only the
test-suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import it.  The GPU library never calls it, and it shares
no code, table or constant with the HIP sources: every format, layout and
codec below is written again here from its definition.

Sources (the five web pages on KV-cache quantization that define the method):

* NInfer KV-cache quantization guide (m.xxqk.cn/news/579065): the paged
  cache with 64-token pages and independent K/V encodings, the per-token
  byte table at head_dim 256, and the five formats BF16, INT8-G64,
  FP8-E4M3 row-256, NVFP4-G16 and K8V4 (section on the five formats).
* TokenSpeed quantization article (gsyq.cn/news/441801), section on the
  ``--kv-cache-dtype`` options: ``fp8_e4m3`` with unit scale and ``mxfp8``
  with one UE8M0 scale per 32 head_dim elements and 128-token blocks.
* Qwen3.8-27B-NVFP4 FP8-KV article (lpnh.cn/news/1821634), section on the
  memory halving: the per-tensor symmetric FP8 ``kv_cache_scheme``; and the
  MTP section (several query tokens per step).
* llama.cpp FP8 KV-cache article (zicq.com), section on why the KV cache is
  compressed: the M_KV size formula.

Where the pages are silent the plainest reading is taken and the docstring
that relies on it says so.  The independent checks that pin each function
live in ``tests/test_oracle_*.py``.
"""

from . import scalar, hadamard, formats, layout, attention  # noqa: F401
