"""Seeded synthetic workloads shaped like the pages' decode scenarios.

This module only draws inputs (queries, keys, values, lengths, page tables);
it holds none of the quantization or attention arithmetic.  Both the GPU
library's callers and the CPU oracle are fed from it.

Recipe:

* host RNG ``numpy.random.default_rng(1000 + config)`` draws, in order, the
  4 special K channels, the sequence lengths, and one global permutation of
  the pool's pages (logical pages of all sequences, concatenated, are
  mapped through it);
* a torch generator on the target device, seeded ``1000 + config``, draws
  q, then K, then V as float32 N(0, 1) and rounds them to bfloat16 (RNE);
* K's 4 special channels are multiplied by 20 (configs 1-4: "outlier
  channels") or replaced by Student-t(3) draws (config 5);
* the softmax scale is 1 / sqrt(head_dim);
* the per-tensor FP8 scale, when calibrated, is fl32(amax|tensor| / 448);
  the per-tensor scale of two-level NVFP4 planes, when asked for, is
  fl32(amax|tensor| / 2688) (6 x 448: the largest E2M1 code times the largest
  UE4M3 scale).

The shapes come from the decode scenarios the pages discuss: GQA with 24
query / 4 KV heads at head_dim 256 and long contexts (NInfer guide, Qwen
FP8-KV article: 262,144-token context), MHA with 128-token blocks for
mxfp8 (TokenSpeed article), and several query tokens per step (MTP).
"""

from dataclasses import dataclass, field
import math

import numpy as np
import torch

FORMAT_IDS = {"BF16": 0, "INT8_G64": 1, "FP8_ROW": 2, "NVFP4_G16": 3, "K8V4": 4, "MXFP8": 5, "FP8_TENSOR": 6, "MXFP4": 7}

CONFIGS = {
    1: dict(name="tiny decode", B=1, H_q=4, H_kv=2, D=256, n_q=1, P=64,
            lengths=("fixed", 1024), k_special="outlier", formats=["BF16", "FP8_ROW"]),
    2: dict(name="batched decode", B=32, H_q=24, H_kv=4, D=256, n_q=1, P=64,
            lengths=("uniform", 8192, 32768), k_special="outlier",
            formats=["INT8_G64", "FP8_ROW", "FP8_TENSOR"]),
    3: dict(name="long-context decode", B=1, H_q=24, H_kv=4, D=256, n_q=1, P=64,
            lengths=("fixed", 262144), k_special="outlier", formats=["NVFP4_G16"]),
    "3b": dict(name="long-context decode, batch 8", B=8, H_q=24, H_kv=4, D=256, n_q=1, P=64,
               lengths=("fixed", 65536), k_special="outlier", formats=["NVFP4_G16"]),
    4: dict(name="mixed-length decode", B=64, H_q=24, H_kv=4, D=256, n_q=1, P=64,
            lengths=("loguniform", 1024, 131072), k_special="outlier", formats=["K8V4"],
            append_chunk=2048),
    5: dict(name="multi-token (MTP) decode", B=256, H_q=32, H_kv=32, D=128, n_q=4, P=128,
            lengths=("fixed", 4096), k_special="student_t3", formats=["MXFP8"]),
}


def _seed(config):
    return 1000 + (3 if config == "3b" else int(config))


@dataclass
class Case:
    config: object
    fmt: int
    D: int
    P: int
    B: int
    H_q: int
    H_kv: int
    n_q: int
    seq_lens: np.ndarray          # [B] int32, includes the n_q newest tokens
    block_table: np.ndarray       # [B, max_pages] int32 (unused entries 0)
    num_pages: int
    q: torch.Tensor               # [B, n_q, H_q, D] bfloat16
    k: torch.Tensor               # [T, H_kv, D] bfloat16, T = sum(seq_lens)
    v: torch.Tensor
    slot_mapping: torch.Tensor    # [T] int32
    softmax_scale: float
    k_scale: float = 1.0
    v_scale: float = 1.0
    token_seq: np.ndarray = field(default=None)   # [T] sequence of each row
    token_pos: np.ndarray = field(default=None)   # [T] position in its sequence
    reserve: int = 0                              # token slots with pages beyond seq_lens

    @property
    def max_pages(self):
        return self.block_table.shape[1]


def _lengths(spec, B, rng):
    if spec[0] == "fixed":
        return np.full(B, spec[1], dtype=np.int64)
    if spec[0] == "uniform":
        return rng.integers(spec[1], spec[2] + 1, size=B)
    if spec[0] == "loguniform":
        return np.floor(np.exp(rng.uniform(math.log(spec[1]), math.log(spec[2]), size=B))).astype(np.int64)
    raise ValueError(spec)


def _bf16_normal(shape, gen, device):
    return torch.randn(shape, generator=gen, device=device, dtype=torch.float32)


def make_case(config, fmt, device="cpu", B=None, lengths=None, n_q=None, extra_pages=0,
              calibrate_tensor_scale=True, reserve=0, two_level=False, H_q=None, H_kv=None):
    """Draw one decode workload.

    ``B``/``lengths`` override the config's batch and lengths (lengths may be
    an explicit list, or a spec tuple) so that the same recipe yields small
    cases the oracle finishes quickly.  ``reserve`` extra token slots per
    sequence are given pages (for later appends) without being drawn.
    ``two_level`` calibrates the per-tensor scales of the NVFP4 planes
    (NVFP4_G16's K and V, K8V4's V).  ``H_q``/``H_kv`` override the head
    counts (other query-group shapes on the same recipe).
    """
    cfg = CONFIGS[config]
    fmt_id = FORMAT_IDS[fmt] if isinstance(fmt, str) else int(fmt)
    B = cfg["B"] if B is None else B
    n_q = cfg["n_q"] if n_q is None else n_q
    D, P = cfg["D"], cfg["P"]
    H_q = cfg["H_q"] if H_q is None else H_q
    H_kv = cfg["H_kv"] if H_kv is None else H_kv
    rng = np.random.default_rng(_seed(config))
    special = rng.choice(D, size=4, replace=False)
    if lengths is None:
        lens = _lengths(cfg["lengths"], B, rng)
    elif isinstance(lengths, tuple):
        lens = _lengths(lengths, B, rng)
    else:
        lens = np.asarray(lengths, dtype=np.int64)
        assert len(lens) == B
    npg = np.array([max(1, -(-(int(L) + reserve) // P)) for L in lens])
    total = int(npg.sum()) + extra_pages
    perm = rng.permutation(total)
    maxp = int(npg.max())
    bt = np.zeros((B, maxp), dtype=np.int32)
    k0 = 0
    for b in range(B):
        bt[b, :npg[b]] = perm[k0:k0 + npg[b]]
        k0 += npg[b]
    T = int(lens.sum())
    gen = torch.Generator(device=device)
    gen.manual_seed(_seed(config))
    q = _bf16_normal((B, n_q, H_q, D), gen, device).to(torch.bfloat16)
    k = _bf16_normal((T, H_kv, D), gen, device)
    sp = torch.as_tensor(special, device=device)
    if cfg["k_special"] == "outlier":
        k[:, :, sp] *= 20.0
    else:  # Student-t(3) = z / sqrt(chi2_3 / 3)
        z = _bf16_normal((T, H_kv, 4), gen, device)
        w = (_bf16_normal((T, H_kv, 4, 3), gen, device) ** 2).sum(-1)
        k[:, :, sp] = z / torch.sqrt(w / 3.0)
    k = k.to(torch.bfloat16)
    v = _bf16_normal((T, H_kv, D), gen, device).to(torch.bfloat16)
    seq = np.repeat(np.arange(B), lens)
    pos = np.concatenate([np.arange(L) for L in lens]) if T else np.zeros(0, np.int64)
    slots = bt[seq, pos // P].astype(np.int64) * P + pos % P
    k_scale = v_scale = 1.0
    if fmt_id == FORMAT_IDS["FP8_TENSOR"] and calibrate_tensor_scale and T:
        k_scale = float(np.float32(k.float().abs().max().item()) / np.float32(448.0))
        v_scale = float(np.float32(v.float().abs().max().item()) / np.float32(448.0))
    if two_level and T and fmt_id in (FORMAT_IDS["NVFP4_G16"], FORMAT_IDS["K8V4"]):
        if fmt_id == FORMAT_IDS["NVFP4_G16"]:
            k_scale = float(np.float32(k.float().abs().max().item()) / np.float32(2688.0))
        v_scale = float(np.float32(v.float().abs().max().item()) / np.float32(2688.0))
    return Case(config, fmt_id, D, P, B, H_q, H_kv, n_q, lens.astype(np.int32), bt, total,
                q, k, v, torch.as_tensor(slots.astype(np.int32), device=device),
                1.0 / math.sqrt(D), k_scale, v_scale, seq, pos, reserve)


def append_chunk(case, chunk, device=None):
    """New K/V rows for ``chunk`` tokens per sequence, placed right after the
    cached tokens (positions L_b .. L_b + chunk - 1); the case must have been
    made with ``reserve >= chunk``.  Returns (k, v, slot_mapping)."""
    device = device or case.k.device
    gen = torch.Generator(device=device)
    gen.manual_seed(_seed(case.config) + 7)
    T = case.B * chunk
    k = _bf16_normal((T, case.H_kv, case.D), gen, device).to(torch.bfloat16)
    v = _bf16_normal((T, case.H_kv, case.D), gen, device).to(torch.bfloat16)
    seq = np.repeat(np.arange(case.B), chunk)
    pos = case.seq_lens[seq].astype(np.int64) + np.tile(np.arange(chunk), case.B)
    if chunk > case.reserve:
        raise ValueError("the case has pages reserved for %d appended tokens, not %d" % (case.reserve, chunk))
    slots = case.block_table[seq, pos // case.P].astype(np.int64) * case.P + pos % case.P
    return k, v, torch.as_tensor(slots.astype(np.int32), device=device)


def bf16_bits(t):
    """bfloat16 tensor -> numpy uint16 bit patterns (host copy)."""
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
