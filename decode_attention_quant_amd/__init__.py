"""Python binding of the kvq C ABI (libkvq.so, HIP for gfx950).

Argument marshalling only: every step of quantize-append, decode attention
and page dequantization runs in the library's HIP kernels.  torch tensors
are used for device memory and streams; their data pointers and the current
HIP stream are passed straight through.  If the library has not been built
the import still works, but every call raises (there is no fallback).
"""

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libkvq.so")

FORMATS = {"BF16": 0, "INT8_G64": 1, "FP8_ROW": 2, "NVFP4_G16": 3, "K8V4": 4, "MXFP8": 5, "FP8_TENSOR": 6,
           "MXFP4": 7}
FORMAT_NAMES = {v: k for k, v in FORMATS.items()}
DEQUANT_STORED_DOMAIN = 1
SPLIT_WRITE_WHOLE_UNITS = 1
SPLIT_Q_MXFP8 = 2  # MXFP8 caches: q rounded to MXFP8, Q.K on the block-scaled fp8 MFMA

STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported", 3: "workspace too small", 4: "HIP runtime error"}

EXPORTS = [
    "kvq_page_bytes", "kvq_quantize_append", "kvq_decode_workspace_size", "kvq_decode_attention",
    "kvq_decode_split", "kvq_decode_combine", "kvq_decode_plan", "kvq_dequant_page", "kvq_status_string",
    "kvq_decode_step", "kvq_decode_step_split", "kvq_prefill_attention",
]


class KvqError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__("%s: %s (status %d)" % (where, STATUS.get(status, "?"), status))


class CacheDesc(ctypes.Structure):
    _fields_ = [("format", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("num_pages", ctypes.c_int64),
                ("k_scale", ctypes.c_float), ("v_scale", ctypes.c_float)]


_lib = None


def library():
    """Load libkvq.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libkvq.so is not built; run `python -m decode_attention_quant_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        P, I32, I64, SZ, F = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float
        D = ctypes.POINTER(CacheDesc)
        sig = {
            "kvq_page_bytes": [D, ctypes.POINTER(SZ)],
            "kvq_quantize_append": [D, P, P, P, I64, P, P],
            "kvq_decode_workspace_size": [D, I32, I32, I32, I32, I32, ctypes.POINTER(SZ)],
            "kvq_decode_attention": [D, P, P, I32, I32, I32, P, I32, P, F, P, P, P, SZ, P],
            "kvq_decode_split": [D, P, P, I32, I32, I32, P, I32, P, F, I32, I32, P, P, P, SZ, P],
            "kvq_decode_step": [D, P, P, P, P, I32, I32, I32, P, I32, P, F, P, P, P, SZ, P],
            "kvq_decode_step_split": [D, P, P, P, P, I32, I32, I32, P, I32, P, F, I32, I32, P, P, P, SZ, P],
            "kvq_prefill_attention": [D, P, P, I32, I32, I32, P, I32, P, F, P, P, P],
            "kvq_decode_combine": [D, I32, I32, I32, I32, P, I32, I32, P, SZ, P, P, P],
            "kvq_decode_plan": [D, I32, I32, I32, I32, ctypes.POINTER(I32), ctypes.POINTER(I32)],
            "kvq_dequant_page": [D, P, I64, I32, P, P, P],
        }
        for name, args in sig.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = ctypes.c_int
        lib.kvq_status_string.argtypes = [ctypes.c_int]
        lib.kvq_status_string.restype = ctypes.c_char_p
        _lib = lib
    return _lib


def _check(status, where):
    if status != 0:
        raise KvqError(status, where)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def desc(fmt, head_dim, page_size, num_kv_heads, num_pages, k_scale=1.0, v_scale=1.0):
    f = FORMATS[fmt] if isinstance(fmt, str) else int(fmt)
    return CacheDesc(f, head_dim, page_size, num_kv_heads, num_pages, k_scale, v_scale)


def page_bytes(d):
    out = ctypes.c_size_t()
    _check(library().kvq_page_bytes(ctypes.byref(d), ctypes.byref(out)), "kvq_page_bytes")
    return out.value


def alloc_pool(d, device="cuda", fill=0xFF):
    """A 256-byte aligned uint8 pool of num_pages pages (torch owns it)."""
    n = page_bytes(d) * d.num_pages
    return torch.full((n,), fill, dtype=torch.uint8, device=device)


def _need(t, dtype, name):
    if not t.is_cuda or t.dtype != dtype or not t.is_contiguous():
        raise ValueError("%s must be a contiguous CUDA tensor of %s" % (name, dtype))


def quantize_append(d, pool, k, v, slot_mapping, stream=None):
    """Encode bf16 K/V [T][H_kv][D] into the pool at slot_mapping[T] (int32)."""
    _need(pool, torch.uint8, "pool")
    _need(k, torch.bfloat16, "k")
    _need(v, torch.bfloat16, "v")
    _need(slot_mapping, torch.int32, "slot_mapping")
    T = k.shape[0]
    _check(library().kvq_quantize_append(ctypes.byref(d), _ptr(pool), _ptr(k), _ptr(v), T, _ptr(slot_mapping),
                                         _stream(stream)), "kvq_quantize_append")


def workspace_size(d, batch, n_q, num_q_heads, max_pages, num_workgroups=0):
    out = ctypes.c_size_t()
    _check(library().kvq_decode_workspace_size(ctypes.byref(d), batch, n_q, num_q_heads, max_pages,
                                               num_workgroups, ctypes.byref(out)), "kvq_decode_workspace_size")
    return out.value


def decode_plan(d, batch, n_q, num_q_heads, max_pages):
    """(split workgroups, partial slots) that decode_attention uses."""
    nwg, slots = ctypes.c_int32(), ctypes.c_int32()
    _check(library().kvq_decode_plan(ctypes.byref(d), batch, n_q, num_q_heads, max_pages, ctypes.byref(nwg),
                                     ctypes.byref(slots)), "kvq_decode_plan")
    return nwg.value, slots.value


def alloc_workspace(nbytes, device="cuda"):
    # torch's caching allocator returns 256-byte aligned blocks
    return torch.empty((max(nbytes, 256),), dtype=torch.uint8, device=device)


def decode_attention(d, pool, q, block_table, seq_lens, softmax_scale, out=None, lse=None, workspace=None,
                     stream=None):
    """out[B][n_q][H_q][D] fp32 (and lse[B][n_q][H_q]) of decode attention."""
    _need(pool, torch.uint8, "pool")
    _need(q, torch.bfloat16, "q")
    _need(block_table, torch.int32, "block_table")
    _need(seq_lens, torch.int32, "seq_lens")
    B, n_q, H_q, D = q.shape
    max_pages = block_table.shape[1]
    if out is None:
        out = torch.empty((B, n_q, H_q, D), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = alloc_workspace(workspace_size(d, B, n_q, H_q, max_pages), q.device)
    _check(library().kvq_decode_attention(
        ctypes.byref(d), _ptr(pool), _ptr(q), B, n_q, H_q, _ptr(block_table), max_pages, _ptr(seq_lens),
        float(softmax_scale), _ptr(out), _ptr(lse), _ptr(workspace), workspace.numel(), _stream(stream)),
        "kvq_decode_attention")
    return out


def decode_step(d, pool, k_new, v_new, q, block_table, seq_lens, softmax_scale, out=None, lse=None, workspace=None,
                stream=None):
    """Append k_new, v_new [B][n_q][H_kv][D] (bf16) at positions seq_lens[b] - n_q + i and run decode attention,
    in one split launch plus the reduce; returns out[B][n_q][H_q][D] fp32."""
    _need(pool, torch.uint8, "pool")
    _need(k_new, torch.bfloat16, "k_new")
    _need(v_new, torch.bfloat16, "v_new")
    _need(q, torch.bfloat16, "q")
    _need(block_table, torch.int32, "block_table")
    _need(seq_lens, torch.int32, "seq_lens")
    B, n_q, H_q, D = q.shape
    if tuple(k_new.shape[:2]) != (B, n_q) or k_new.shape != v_new.shape:
        raise ValueError("k_new and v_new must be [B][n_q][H_kv][D] with q's B and n_q")
    max_pages = block_table.shape[1]
    if out is None:
        out = torch.empty((B, n_q, H_q, D), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = alloc_workspace(workspace_size(d, B, n_q, H_q, max_pages), q.device)
    _check(library().kvq_decode_step(
        ctypes.byref(d), _ptr(pool), _ptr(k_new), _ptr(v_new), _ptr(q), B, n_q, H_q, _ptr(block_table), max_pages,
        _ptr(seq_lens), float(softmax_scale), _ptr(out), _ptr(lse), _ptr(workspace), workspace.numel(),
        _stream(stream)), "kvq_decode_step")
    return out


def decode_step_split(d, pool, k_new, v_new, q, block_table, seq_lens, softmax_scale, workspace, num_workgroups=0,
                      flags=0, out=None, lse=None, stream=None):
    """The fused step's split phase (stores the new tokens, then decodes); finish with decode_combine."""
    B, n_q, H_q, D = q.shape
    _check(library().kvq_decode_step_split(
        ctypes.byref(d), _ptr(pool), _ptr(k_new), _ptr(v_new), _ptr(q), B, n_q, H_q, _ptr(block_table),
        block_table.shape[1], _ptr(seq_lens), float(softmax_scale), num_workgroups, flags, _ptr(out), _ptr(lse),
        _ptr(workspace), workspace.numel(), _stream(stream)), "kvq_decode_step_split")


def prefill_attention(d, pool, q, block_table, seq_lens, softmax_scale, out=None, lse=None, stream=None):
    """Causal attention of a prefill chunk's queries q[B][n_q][H_q][D] (positions seq_lens[b] - n_q + i, already
    appended) over the cache; returns out[B][n_q][H_q][D] fp32."""
    _need(pool, torch.uint8, "pool")
    _need(q, torch.bfloat16, "q")
    _need(block_table, torch.int32, "block_table")
    _need(seq_lens, torch.int32, "seq_lens")
    B, n_q, H_q, D = q.shape
    if out is None:
        out = torch.empty((B, n_q, H_q, D), dtype=torch.float32, device=q.device)
    _check(library().kvq_prefill_attention(
        ctypes.byref(d), _ptr(pool), _ptr(q), B, n_q, H_q, _ptr(block_table), block_table.shape[1], _ptr(seq_lens),
        float(softmax_scale), _ptr(out), _ptr(lse), _stream(stream)), "kvq_prefill_attention")
    return out


def decode_split(d, pool, q, block_table, seq_lens, softmax_scale, workspace, num_workgroups=0, flags=0, out=None,
                 lse=None, stream=None):
    B, n_q, H_q, D = q.shape
    _check(library().kvq_decode_split(
        ctypes.byref(d), _ptr(pool), _ptr(q), B, n_q, H_q, _ptr(block_table), block_table.shape[1],
        _ptr(seq_lens), float(softmax_scale), num_workgroups, flags, _ptr(out), _ptr(lse), _ptr(workspace),
        workspace.numel(), _stream(stream)), "kvq_decode_split")


def decode_combine(d, batch, n_q, num_q_heads, max_pages, seq_lens, workspace, out, lse=None, num_workgroups=0,
                   flags=0, stream=None):
    _check(library().kvq_decode_combine(
        ctypes.byref(d), batch, n_q, num_q_heads, max_pages, _ptr(seq_lens), num_workgroups, flags,
        _ptr(workspace), workspace.numel(), _ptr(out), _ptr(lse), _stream(stream)), "kvq_decode_combine")


def dequant_page(d, pool, page, stored_domain=True, stream=None):
    """fp32 K, V [H_kv][P][D] of one physical page."""
    k = torch.empty((d.num_kv_heads, d.page_size, d.head_dim), dtype=torch.float32, device=pool.device)
    v = torch.empty_like(k)
    _check(library().kvq_dequant_page(ctypes.byref(d), _ptr(pool), int(page),
                                      DEQUANT_STORED_DOMAIN if stored_domain else 0, _ptr(k), _ptr(v),
                                      _stream(stream)), "kvq_dequant_page")
    return k, v
