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
    "kvq_page_bytes", "kvq_quantize_append", "kvq_decode_workspace_size", "kvq_decode_workspace_size_for",
    "kvq_decode_attention", "kvq_decode_attention_noalloc",
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
            "kvq_decode_workspace_size": [D, I32, I32, I32, I32, ctypes.POINTER(SZ)],
            "kvq_decode_workspace_size_for": [D, I32, I32, I32, I32, I32, ctypes.POINTER(SZ)],
            "kvq_decode_attention": [D, P, P, I32, I32, I32, P, I32, P, F, P, P, P, SZ, P],
            "kvq_decode_attention_noalloc": [D, P, P, I32, I32, I32, P, I32, P, F, P, P, P],
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


def _need(t, dtype, name, shape=None):
    """Check a tensor before its pointer crosses the boundary: dtype, shape
    (entries that are not None) and contiguity.  A mismatch raises ValueError
    and nothing is launched: the kernels trust these sizes.  Where the
    tensors live is checked afterwards, for all of them at once (_placed)."""
    if not isinstance(t, torch.Tensor):
        raise ValueError("%s must be a torch tensor" % name)
    if t.dtype != dtype:
        raise ValueError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if shape is not None:
        if t.dim() != len(shape) or any(w is not None and int(n) != int(w) for n, w in zip(t.shape, shape)):
            raise ValueError("%s must have shape %s, got %s" % (
                name, tuple("*" if w is None else int(w) for w in shape), tuple(t.shape)))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def _placed(**tensors):
    """Every tensor given (None entries skipped) on one GPU."""
    dev = None
    for name, t in tensors.items():
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("%s must be a CUDA tensor" % name)
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError("%s is on %s, other arguments on %s" % (name, t.device, dev))


def _need_pool(d, pool):
    """The pool: a 1-D uint8 tensor holding num_pages whole pages."""
    if not isinstance(pool, torch.Tensor) or pool.dim() != 1:
        raise ValueError("pool must be a 1-D uint8 tensor")
    _need(pool, torch.uint8, "pool")
    need = page_bytes(d) * d.num_pages
    if pool.numel() < need:
        raise ValueError("pool holds %d bytes; %d pages of %d bytes need %d" % (
            pool.numel(), d.num_pages, page_bytes(d), need))


def _need_decode(d, pool, q, block_table, seq_lens, out, lse):
    """Shapes of a decode-style call: q [B][n_q][H_q][D] bf16 with D = head_dim
    and H_q a multiple of H_kv, block_table int32 [B][max_pages], seq_lens int32
    [B], out fp32 [B][n_q][H_q][D], lse fp32 [B][n_q][H_q] or None.  Returns
    (B, n_q, H_q, max_pages)."""
    if not isinstance(q, torch.Tensor) or q.dim() != 4:
        raise ValueError("q must be a 4-D tensor [B][n_q][H_q][D]")
    B, n_q, H_q, D = (int(x) for x in q.shape)
    if D != d.head_dim:
        raise ValueError("q's last dimension is %d, the cache's head_dim %d" % (D, d.head_dim))
    if H_q % d.num_kv_heads != 0:
        raise ValueError("num_q_heads %d is not a multiple of num_kv_heads %d" % (H_q, d.num_kv_heads))
    _need_pool(d, pool)
    _need(q, torch.bfloat16, "q")
    if not isinstance(block_table, torch.Tensor) or block_table.dim() != 2:
        raise ValueError("block_table must be a 2-D int32 tensor [B][max_pages]")
    _need(block_table, torch.int32, "block_table", (B, None))
    _need(seq_lens, torch.int32, "seq_lens", (B,))
    if out is not None:
        _need(out, torch.float32, "out", (B, n_q, H_q, D))
    if lse is not None:
        _need(lse, torch.float32, "lse", (B, n_q, H_q))
    return B, n_q, H_q, int(block_table.shape[1])


def _need_new_tokens(d, k_new, v_new, B, n_q):
    _need(k_new, torch.bfloat16, "k_new", (B, n_q, d.num_kv_heads, d.head_dim))
    _need(v_new, torch.bfloat16, "v_new", (B, n_q, d.num_kv_heads, d.head_dim))


def _need_workspace(workspace):
    if not isinstance(workspace, torch.Tensor) or workspace.dim() != 1:
        raise ValueError("workspace must be a 1-D uint8 tensor")
    _need(workspace, torch.uint8, "workspace")


def quantize_append(d, pool, k, v, slot_mapping, stream=None):
    """Encode bf16 K/V [T][H_kv][D] into the pool at slot_mapping[T] (int32)."""
    _need_pool(d, pool)
    if not isinstance(k, torch.Tensor) or k.dim() != 3:
        raise ValueError("k must be a 3-D tensor [T][H_kv][D]")
    T = int(k.shape[0])
    _need(k, torch.bfloat16, "k", (T, d.num_kv_heads, d.head_dim))
    _need(v, torch.bfloat16, "v", (T, d.num_kv_heads, d.head_dim))
    _need(slot_mapping, torch.int32, "slot_mapping", (T,))
    _placed(pool=pool, k=k, v=v, slot_mapping=slot_mapping)
    _check(library().kvq_quantize_append(ctypes.byref(d), _ptr(pool), _ptr(k), _ptr(v), T, _ptr(slot_mapping),
                                         _stream(stream)), "kvq_quantize_append")


def workspace_size(d, batch, n_q, num_q_heads, max_pages, num_workgroups=0):
    """Workspace bytes of the planned split (num_workgroups = 0) or of a forced one."""
    out = ctypes.c_size_t()
    if num_workgroups == 0:
        _check(library().kvq_decode_workspace_size(ctypes.byref(d), batch, n_q, num_q_heads, max_pages,
                                                   ctypes.byref(out)), "kvq_decode_workspace_size")
    else:
        _check(library().kvq_decode_workspace_size_for(ctypes.byref(d), batch, n_q, num_q_heads, max_pages,
                                                       num_workgroups, ctypes.byref(out)),
               "kvq_decode_workspace_size_for")
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
    B, n_q, H_q, max_pages = _need_decode(d, pool, q, block_table, seq_lens, out, lse)
    if workspace is not None:
        _need_workspace(workspace)
    _placed(pool=pool, q=q, block_table=block_table, seq_lens=seq_lens, out=out, lse=lse, workspace=workspace)
    if out is None:
        out = torch.empty((B, n_q, H_q, d.head_dim), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = alloc_workspace(workspace_size(d, B, n_q, H_q, max_pages), q.device)
    _check(library().kvq_decode_attention(
        ctypes.byref(d), _ptr(pool), _ptr(q), B, n_q, H_q, _ptr(block_table), max_pages, _ptr(seq_lens),
        float(softmax_scale), _ptr(out), _ptr(lse), _ptr(workspace), workspace.numel(), _stream(stream)),
        "kvq_decode_attention")
    return out


NOALLOC_SCRATCH_BYTES = 64 << 20  # KVQ_NOALLOC_SCRATCH_BYTES


def decode_attention_noalloc(d, pool, q, block_table, seq_lens, softmax_scale, out, lse=None, stream=None):
    """decode_attention with the library's own device scratch as the workspace
    (the caller allocates nothing but out/lse, which it passes in)."""
    B, n_q, H_q, max_pages = _need_decode(d, pool, q, block_table, seq_lens, out, lse)
    if out is None:
        raise ValueError("out must be given")
    _placed(pool=pool, q=q, block_table=block_table, seq_lens=seq_lens, out=out, lse=lse)
    _check(library().kvq_decode_attention_noalloc(
        ctypes.byref(d), _ptr(pool), _ptr(q), B, n_q, H_q, _ptr(block_table), max_pages, _ptr(seq_lens),
        float(softmax_scale), _ptr(out), _ptr(lse), _stream(stream)), "kvq_decode_attention_noalloc")


def decode_step(d, pool, k_new, v_new, q, block_table, seq_lens, softmax_scale, out=None, lse=None, workspace=None,
                stream=None):
    """Append k_new, v_new [B][n_q][H_kv][D] (bf16) at positions seq_lens[b] - n_q + i and run decode attention,
    in one split launch plus the reduce; returns out[B][n_q][H_q][D] fp32."""
    B, n_q, H_q, max_pages = _need_decode(d, pool, q, block_table, seq_lens, out, lse)
    _need_new_tokens(d, k_new, v_new, B, n_q)
    if workspace is not None:
        _need_workspace(workspace)
    _placed(pool=pool, k_new=k_new, v_new=v_new, q=q, block_table=block_table, seq_lens=seq_lens, out=out, lse=lse,
            workspace=workspace)
    if out is None:
        out = torch.empty((B, n_q, H_q, d.head_dim), dtype=torch.float32, device=q.device)
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
    B, n_q, H_q, max_pages = _need_decode(d, pool, q, block_table, seq_lens, out, lse)
    _need_new_tokens(d, k_new, v_new, B, n_q)
    _need_workspace(workspace)
    _placed(pool=pool, k_new=k_new, v_new=v_new, q=q, block_table=block_table, seq_lens=seq_lens, out=out, lse=lse,
            workspace=workspace)
    _check(library().kvq_decode_step_split(
        ctypes.byref(d), _ptr(pool), _ptr(k_new), _ptr(v_new), _ptr(q), B, n_q, H_q, _ptr(block_table),
        max_pages, _ptr(seq_lens), float(softmax_scale), num_workgroups, flags, _ptr(out), _ptr(lse),
        _ptr(workspace), workspace.numel(), _stream(stream)), "kvq_decode_step_split")


def prefill_attention(d, pool, q, block_table, seq_lens, softmax_scale, out=None, lse=None, stream=None):
    """Causal attention of a prefill chunk's queries q[B][n_q][H_q][D] (positions seq_lens[b] - n_q + i, already
    appended) over the cache; returns out[B][n_q][H_q][D] fp32."""
    B, n_q, H_q, max_pages = _need_decode(d, pool, q, block_table, seq_lens, out, lse)
    _placed(pool=pool, q=q, block_table=block_table, seq_lens=seq_lens, out=out, lse=lse)
    if out is None:
        out = torch.empty((B, n_q, H_q, d.head_dim), dtype=torch.float32, device=q.device)
    _check(library().kvq_prefill_attention(
        ctypes.byref(d), _ptr(pool), _ptr(q), B, n_q, H_q, _ptr(block_table), max_pages, _ptr(seq_lens),
        float(softmax_scale), _ptr(out), _ptr(lse), _stream(stream)), "kvq_prefill_attention")
    return out


def decode_split(d, pool, q, block_table, seq_lens, softmax_scale, workspace, num_workgroups=0, flags=0, out=None,
                 lse=None, stream=None):
    """The split phase of decode attention (partials into the workspace); finish with decode_combine."""
    B, n_q, H_q, max_pages = _need_decode(d, pool, q, block_table, seq_lens, out, lse)
    _need_workspace(workspace)
    _placed(pool=pool, q=q, block_table=block_table, seq_lens=seq_lens, out=out, lse=lse, workspace=workspace)
    _check(library().kvq_decode_split(
        ctypes.byref(d), _ptr(pool), _ptr(q), B, n_q, H_q, _ptr(block_table), max_pages,
        _ptr(seq_lens), float(softmax_scale), num_workgroups, flags, _ptr(out), _ptr(lse), _ptr(workspace),
        workspace.numel(), _stream(stream)), "kvq_decode_split")


def decode_combine(d, batch, n_q, num_q_heads, max_pages, seq_lens, workspace, out, lse=None, num_workgroups=0,
                   flags=0, stream=None):
    """Merge the split phase's partials into out[B][n_q][H_q][D] (and lse)."""
    if num_q_heads % d.num_kv_heads != 0:
        raise ValueError("num_q_heads %d is not a multiple of num_kv_heads %d" % (num_q_heads, d.num_kv_heads))
    _need_workspace(workspace)
    _need(seq_lens, torch.int32, "seq_lens", (batch,))
    _need(out, torch.float32, "out", (batch, n_q, num_q_heads, d.head_dim))
    if lse is not None:
        _need(lse, torch.float32, "lse", (batch, n_q, num_q_heads))
    _placed(workspace=workspace, seq_lens=seq_lens, out=out, lse=lse)
    _check(library().kvq_decode_combine(
        ctypes.byref(d), batch, n_q, num_q_heads, max_pages, _ptr(seq_lens), num_workgroups, flags,
        _ptr(workspace), workspace.numel(), _ptr(out), _ptr(lse), _stream(stream)), "kvq_decode_combine")


def dequant_page(d, pool, page, stored_domain=True, stream=None):
    """fp32 K, V [H_kv][P][D] of one physical page."""
    _need_pool(d, pool)
    if not 0 <= int(page) < d.num_pages:
        raise ValueError("page %d is outside the pool's %d pages" % (int(page), d.num_pages))
    _placed(pool=pool)
    k = torch.empty((d.num_kv_heads, d.page_size, d.head_dim), dtype=torch.float32, device=pool.device)
    v = torch.empty_like(k)
    _check(library().kvq_dequant_page(ctypes.byref(d), _ptr(pool), int(page),
                                      DEQUANT_STORED_DOMAIN if stored_domain else 0, _ptr(k), _ptr(v),
                                      _stream(stream)), "kvq_dequant_page")
    return k, v
