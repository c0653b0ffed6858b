"""ctypes binding of libnvfp4kv_probe.so (include/nvfp4kv_probe.h): the
benchmark's read-only stream, a measurement aid and not an operation of the
NVFP4 KV cache."""
from __future__ import annotations

import ctypes
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libnvfp4kv_probe.so")
EXPORTS = ["nvfp4kv_probe_read_pages", "nvfp4kv_probe_read_stream"]
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
        fn = lib.nvfp4kv_probe_read_pages
        fn.restype = ctypes.c_int32
        fn.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int32,
                       ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_int32,
                       ctypes.c_int32, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
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


def read_pages(pool: torch.Tensor, block_table: torch.Tensor, seq_lens: torch.Tensor, sink: torch.Tensor,
               splits: int) -> None:
    """Read every page slab a decode batch reads from a pool view (num_blocks,
    2, block_size, num_kv_heads, row) whose page rows are contiguous, in
    `splits` ranges per (sequence, kv head); sink: int32, 4 per workgroup."""
    nb, _, bs, hkv, row = pool.shape
    st = [x * pool.element_size() for x in pool.stride()]
    if st[2] != row * pool.element_size() or st[4] != pool.element_size():
        raise ValueError("read_pages needs contiguous page rows (HND layout)")
    grid = seq_lens.numel() * hkv * splits
    if not (block_table.dtype == torch.int32 and seq_lens.dtype == torch.int32 and block_table.is_contiguous()
            and block_table.shape[0] >= seq_lens.numel() and sink.dtype == torch.int32 and sink.numel() >= 4 * grid):
        raise ValueError("read_pages: int32 contiguous block table and lengths, int32 sink of 4 per workgroup")
    rc = library().nvfp4kv_probe_read_pages(
        ctypes.c_void_p(pool.data_ptr()), nb, st[0], st[1], st[3], bs * row * pool.element_size(), bs, hkv,
        ctypes.c_void_p(block_table.data_ptr()), block_table.shape[1], ctypes.c_void_p(seq_lens.data_ptr()),
        seq_lens.numel(), splits, ctypes.c_void_p(sink.data_ptr()), sink.numel() * 4,
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    if rc != 0:
        raise RuntimeError(f"nvfp4kv_probe_read_pages returned {rc}")
