"""ctypes binding of ``libmoe_probe.so`` (``include/moe_probe.h``): the
bandwidth probes the benchmark times beside the routing path. Argument
marshalling only; raises if the library is not built."""
from __future__ import annotations

import ctypes
import os

import torch

from .binding import MoeError, _ptr, _stream

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libmoe_probe.so")
_lib = None


def load_library():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError("libmoe_probe.so is not built (run __graft_entry__.build())")
    lib = ctypes.CDLL(_LIB_PATH)
    p, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    lib.moe_probe_read.argtypes = [p, sz, p, p]
    lib.moe_probe_read.restype = ctypes.c_int
    lib.moe_probe_write.argtypes = [p, sz, ctypes.c_uint32, i32, p]
    lib.moe_probe_write.restype = ctypes.c_int
    lib.moe_probe_gather.argtypes = [p, p, i64, i32, i64, p, p]
    lib.moe_probe_gather.restype = ctypes.c_int
    lib.moe_probe_empty.argtypes = [i32, p]
    lib.moe_probe_empty.restype = ctypes.c_int
    lib.moe_probe_consume.argtypes = [p, sz, p, p]
    lib.moe_probe_consume.restype = ctypes.c_int
    _lib = lib
    return lib


def _check(fn, st):
    if st != 0:
        raise MoeError(fn, st)


def read(src: torch.Tensor, sink: torch.Tensor, stream=None):
    """Stream every byte of src once (finalize's loads)."""
    st = load_library().moe_probe_read(_ptr(src), src.numel() * src.element_size(), _ptr(sink),
                                       _stream(stream, src))
    _check("moe_probe_read", st)


def write(dst: torch.Tensor, value: int = 0x3F803F80, streaming: bool = False, stream=None):
    """Fill every byte of dst (finalize's stores: non-temporal when
    `streaming`, sc1 otherwise)."""
    st = load_library().moe_probe_write(_ptr(dst), dst.numel() * dst.element_size(),
                                        value & 0xFFFFFFFF, 1 if streaming else 0,
                                        _stream(stream, dst))
    _check("moe_probe_write", st)


def gather(rows: torch.Tensor, restore: torch.Tensor, T: int, K: int, sink: torch.Tensor,
           stream=None):
    """finalize's gather of K rows per token through restore, without stores."""
    st = load_library().moe_probe_gather(_ptr(rows), _ptr(restore), T, K,
                                         rows.shape[1] * rows.element_size(), _ptr(sink),
                                         _stream(stream, rows))
    _check("moe_probe_gather", st)


def empty(workgroups: int = 1, stream=None):
    """A launch of `workgroups` workgroups that do nothing."""
    if stream is None:
        stream = torch.cuda.current_stream()
    st = load_library().moe_probe_empty(int(workgroups), _stream(stream))
    _check("moe_probe_empty", st)


def consume(src: torch.Tensor, sink: torch.Tensor, stream=None):
    """One workgroup reads every byte of src (at most 256 KiB)."""
    st = load_library().moe_probe_consume(_ptr(src), src.numel() * src.element_size(),
                                          _ptr(sink), _stream(stream, src))
    _check("moe_probe_consume", st)
