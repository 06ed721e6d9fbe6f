"""ctypes binding of libkvq_probe.so (include/kvq_probe.h): the GPU's own
streaming-read and matrix-core loop rates, which the benchmark quotes its
rooflines against.  Not part of the attention path."""
from __future__ import annotations

import ctypes
import os

import torch

from ._binding import KvqError, _ptr, _stream

HERE = os.path.dirname(os.path.abspath(__file__))
_lib = None


def _check(status: int) -> None:
    if status != 0:
        raise KvqError(status, "probe call rejected its arguments or failed to launch")


def probe_library_path() -> str:
    return os.path.join(HERE, "libkvq_probe.so")


def load_probe_library():
    global _lib
    if _lib is not None:
        return _lib
    path = probe_library_path()
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with block_quantized_kv_amd/build.py")
    lib = ctypes.CDLL(path)
    P, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    lib.kvq_probe_stream_read.restype = i32
    lib.kvq_probe_stream_read.argtypes = [P, sz, i32, P, P]
    lib.kvq_probe_mfma_f16.restype = i32
    lib.kvq_probe_mfma_f16.argtypes = [i32, i32, P, ctypes.POINTER(ctypes.c_double), P]
    _lib = lib
    return lib


def kvq_probe_stream_read(buf, n_workgroups: int, sink, stream=None) -> None:
    """Streaming read of the whole contiguous device tensor `buf`; sink: int32 [1] device."""
    if not buf.is_cuda or not buf.is_contiguous():
        raise ValueError("buf must be a contiguous device tensor")
    if sink.dtype != torch.int32 or sink.numel() != 1 or not sink.is_cuda:
        raise ValueError("sink: expected a device int32 [1] tensor")
    _check(load_probe_library().kvq_probe_stream_read(_ptr(buf), buf.numel() * buf.element_size(),
                                                      n_workgroups, _ptr(sink), _stream(stream)))


def kvq_probe_mfma_f16(n_workgroups: int, iters: int, sink, stream=None) -> float:
    """Enqueues the matrix-core loop; returns the flop count of the launch."""
    if sink.dtype != torch.int32 or sink.numel() != 1 or not sink.is_cuda:
        raise ValueError("sink: expected a device int32 [1] tensor")
    flop = ctypes.c_double()
    _check(load_probe_library().kvq_probe_mfma_f16(n_workgroups, iters, _ptr(sink), ctypes.byref(flop),
                                                   _stream(stream)))
    return flop.value
