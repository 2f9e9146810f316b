"""Binding of libkvq_probe.so: a streaming read and a copy kernel that
calibrate measurements of the kvq kernels (the reachable HBM read rate,
cache eviction between timed runs, and a known byte count for scaling HBM
byte counters).  Not part of the kvq boundary."""

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(os.path.dirname(HERE), "libkvq_probe.so")
EXPORTS = ["kvq_probe_read", "kvq_probe_read_stream", "kvq_probe_copy"]

_lib = None


def library():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libkvq_probe.so is not built; run `python -m decode_attention_quant_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        P, SZ = ctypes.c_void_p, ctypes.c_size_t
        lib.kvq_probe_read.argtypes = lib.kvq_probe_read_stream.argtypes = [P, SZ, P, P]
        lib.kvq_probe_copy.argtypes = [P, P, SZ, P]
        lib.kvq_probe_read.restype = lib.kvq_probe_read_stream.restype = lib.kvq_probe_copy.restype = ctypes.c_int
        _lib = lib
    return _lib


def _stream(stream):
    return ctypes.c_void_p((stream or torch.cuda.current_stream()).cuda_stream)


def read(buf, sink, stream=None, nontemporal=False):
    """Read every byte of the contiguous device tensor ``buf`` once (plain
    loads, which also evict the caches; or with the non-temporal hint)."""
    fn = library().kvq_probe_read_stream if nontemporal else library().kvq_probe_read
    st = fn(ctypes.c_void_p(buf.data_ptr()), buf.numel() * buf.element_size(), ctypes.c_void_p(sink.data_ptr()),
            _stream(stream))
    if st:
        raise RuntimeError("kvq_probe_read failed (%d)" % st)


def copy(dst, src, stream=None):
    n = src.numel() * src.element_size()
    assert dst.numel() * dst.element_size() >= n
    st = library().kvq_probe_copy(ctypes.c_void_p(dst.data_ptr()), ctypes.c_void_p(src.data_ptr()), n,
                                  _stream(stream))
    if st:
        raise RuntimeError("kvq_probe_copy failed (%d)" % st)
