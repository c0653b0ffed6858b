"""ctypes binding of libnvfp4kv_probe.so (include/nvfp4kv_probe.h): the
benchmark's read-only stream, a measurement aid and not an operation of the
NVFP4 KV cache."""
from __future__ import annotations

import ctypes
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libnvfp4kv_probe.so")
EXPORTS = ["nvfp4kv_probe_read_stream"]
_lib = None


def library():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m bit_quantized_paged_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        fn = lib.nvfp4kv_probe_read_stream
        fn.restype = ctypes.c_int32
        fn.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_int64,
                       ctypes.c_void_p]
        _lib = lib
    return _lib


def read_stream(t: torch.Tensor, nbytes: int, sink: torch.Tensor, grid: int) -> None:
    """Read the first nbytes (a multiple of 16) of device tensor t's storage."""
    if not (t.is_cuda and sink.is_cuda and sink.dtype == torch.int32 and sink.numel() >= 4 * grid):
        raise ValueError("read_stream needs device tensors and an int32 sink of at least 4 * grid entries")
    if nbytes > t.numel() * t.element_size():
        raise ValueError("nbytes exceeds the tensor")
    st = library().nvfp4kv_probe_read_stream(ctypes.c_void_p(t.data_ptr()), nbytes, grid,
                                              ctypes.c_void_p(sink.data_ptr()), sink.numel() * 4,
                                              ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    if st != 0:
        raise RuntimeError(f"nvfp4kv_probe_read_stream returned {st}")
