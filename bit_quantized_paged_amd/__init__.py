"""NVFP4-quantised paged KV cache for AMD Instinct MI355X (gfx950), with FP8
(E4M3FN, E5M2) caches through the same entry points and NVFP4 activation
quantisation.

Thin ctypes binding of ``libnvfp4kv.so`` (built from ``csrc/`` by
``bit_quantized_paged_amd.build``). The functions here only marshal torch
tensors (device memory and the current HIP stream) into the C ABI declared in
``include/nvfp4kv.h``; every step of the computation runs in the HIP kernels.
There is no CPU fallback: without the built library every call raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "NVFP4KVError", "library", "full_dim", "row_bytes", "KV_DTYPES", "kv_dtype_of", "alloc_pool", "append",
    "dequant_paged", "dequant_pages", "qdq", "decode_workspace_size", "prefill_workspace_size", "decode_plan",
    "paged_attention_decode",
    "paged_attention_prefill", "fp8_to_bf16", "quant_activations", "quant_activations_scale_bytes",
    "paged_attention_decode_noalloc",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libnvfp4kv.so")

EXPORTS = [
    "nvfp4_kv_full_dim", "nvfp4_kv_append", "nvfp4_kv_dequant_paged", "nvfp4_kv_dequant_pages", "nvfp4_kv_qdq",
    "nvfp4_paged_attention_decode_workspace_size", "nvfp4_paged_attention_prefill_workspace_size",
    "nvfp4_paged_attention_decode_plan",
    "nvfp4_paged_attention_decode", "nvfp4_paged_attention_decode_fp8", "nvfp4_fp8_to_bf16",
    "nvfp4_paged_attention_decode_noalloc",
    "nvfp4_paged_attention_prefill_fp8",
    "nvfp4_paged_attention_prefill", "nvfp4_quant_activations", "nvfp4_quant_activations_scale_bytes",
    "nvfp4kv_status_string", "nvfp4kv_last_error",
]


class NVFP4KVError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"nvfp4kv status {status}: {message}")
        self.status = status


class CacheDesc(ctypes.Structure):
    _fields_ = [
        ("data", ctypes.c_void_p), ("num_blocks", ctypes.c_int64), ("block_size", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32), ("head_size", ctypes.c_int32), ("kv_dtype", ctypes.c_int32),
        ("stride_block", ctypes.c_int64), ("stride_kv", ctypes.c_int64), ("stride_token", ctypes.c_int64),
        ("stride_head", ctypes.c_int64),
    ]


_lib = None
_P, _I32, _I64, _F32, _SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
_DESC = ctypes.POINTER(CacheDesc)


def library():
    """The loaded libnvfp4kv.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m bit_quantized_paged_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        sig = {
            "nvfp4_kv_full_dim": (_I32, [_I32]),
            "nvfp4_kv_append": (_I32, [_DESC, _P, _I64, _I64, _P, _I64, _I64, _P, _I64, _P, _P, _P]),
            "nvfp4_kv_dequant_paged": (_I32, [_DESC, _P, _I32, _P, _P, _I32, _I32, _P, _P, _P, _P, _I64, _P]),
            "nvfp4_kv_dequant_pages": (_I32, [_DESC, _P, _I32, _P, _P, _P, _I64, _I64, _I64, _I64, _P]),
            "nvfp4_kv_qdq": (_I32, [_P, _I64, _I64, _P, _I64, _I64, _I64, _I32, _I32, _P, _P, _P]),
            "nvfp4_paged_attention_decode_workspace_size": (_SZ, [_I32, _I32, _I32, _I32]),
            "nvfp4_paged_attention_prefill_workspace_size": (_SZ, [_I32]),
            "nvfp4_paged_attention_decode_plan": (_I32, [_I32, _I32, _I32, _I32, _I32, _I32, _I32]),
            "nvfp4_paged_attention_decode": (_I32, [_DESC, _P, _I64, _I64, _I32, _P, _I32, _P, _I32, _I32, _P, _P,
                                                    _F32, _P, _P, _SZ, _P]),
            "nvfp4_paged_attention_decode_fp8": (_I32, [_DESC, _P, _I64, _I64, _I32, _P, _I32, _P, _I32, _I32, _P,
                                                        _P, _F32, _P, _P, _P, _SZ, _P]),
            "nvfp4_fp8_to_bf16": (_I32, [_P, _I64, _P, _P, _P]),
            "nvfp4_paged_attention_decode_noalloc": (_I32, [_DESC, _P, _I64, _I64, _I32, _P, _I32, _P, _I32, _I32,
                                                            _P, _P, _F32, _P, _P]),
            "nvfp4_paged_attention_prefill_fp8": (_I32, [_DESC, _P, _I64, _I64, _I32, _P, _I32, _I32, _P, _I32, _P,
                                                         _I32, _I32, _P, _P, _F32, _I32, _P, _P, _P, _SZ, _P]),
            "nvfp4_paged_attention_prefill": (_I32, [_DESC, _P, _I64, _I64, _I32, _P, _I32, _I32, _P, _I32, _P, _I32,
                                                     _I32, _P, _P, _F32, _I32, _P, _P, _SZ, _P]),
            "nvfp4_quant_activations": (_I32, [_P, _I64, _I64, _I32, _P, _I32, _P, _P, _P]),
            "nvfp4_quant_activations_scale_bytes": (_I64, [_I64, _I32, _I32]),
            "nvfp4kv_status_string": (ctypes.c_char_p, [_I32]),
            "nvfp4kv_last_error": (ctypes.c_char_p, []),
        }
        for name, (res, args) in sig.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def _check(status: int) -> None:
    if status != 0:
        lib = library()
        raise NVFP4KVError(status, lib.nvfp4kv_last_error().decode() or lib.nvfp4kv_status_string(status).decode())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


# Every size the kernels read or write through a pointer is checked here,
# against the pool descriptor and the batch size, before anything reaches the
# C ABI (which sees pointers, not shapes). Checks take the order dtype,
# shape, layout, device, so a mis-sized tensor is reported as such wherever
# it lives.
def _meta(t, name, dtype):
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")


def _shape(t, name, want):
    """want: a tuple of ints (None matches any size)."""
    got = tuple(t.shape)
    if len(got) != len(want) or any(w is not None and g != w for g, w in zip(got, want)):
        shown = tuple("*" if w is None else w for w in want)
        raise ValueError(f"{name} must have shape {shown}, got {got}")


def _scalar(t, name):
    _meta(t, name, torch.float32)
    if t.numel() < 1:
        raise ValueError(f"{name} must hold one float32 value")


def _devices(*named):
    for t, name in named:
        if t is not None and not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")


def full_dim(head_size: int) -> int:
    return int(library().nvfp4_kv_full_dim(head_size))


# Cache formats and the torch dtype of their pools [P40177 "Key source
# snippets", get_dtype_for_flashinfer: fp8_e4m3 -> float8_e4m3fn, fp8_e5m2 ->
# float8_e5m2, nvfp4 -> uint8 holding packed FP4 data and FP8 block scales].
KV_NVFP4, KV_FP8_E4M3, KV_FP8_E5M2 = 0, 1, 2
KV_DTYPES = {"nvfp4": (KV_NVFP4, torch.uint8), "fp8_e4m3": (KV_FP8_E4M3, torch.float8_e4m3fn),
             "fp8_e5m2": (KV_FP8_E5M2, torch.float8_e5m2)}
_KV_OF_TORCH = {dt: code for code, dt in KV_DTYPES.values()}


def row_bytes(head_size: int, kv_dtype: str = "nvfp4") -> int:
    return head_size // 2 + head_size // 16 if kv_dtype == "nvfp4" else head_size


def alloc_pool(num_blocks: int, block_size: int, num_kv_heads: int, head_size: int,
               layout: str = "HND", device="cuda", kv_dtype: str = "nvfp4") -> torch.Tensor:
    """Zeroed pool, returned as the logical view (num_blocks, 2, block_size,
    num_kv_heads, row bytes) in the torch dtype of its format (uint8 for
    NVFP4, float8_e4m3fn / float8_e5m2 for FP8). ``layout`` picks the
    physical order: "HND" stores (num_blocks, 2, num_kv_heads, block_size, row)."""
    fd = row_bytes(head_size, kv_dtype)
    dt = KV_DTYPES[kv_dtype][1]
    if layout == "HND":
        return torch.zeros((num_blocks, 2, num_kv_heads, block_size, fd), dtype=dt,
                           device=device).permute(0, 1, 3, 2, 4)
    if layout == "NHD":
        return torch.zeros((num_blocks, 2, block_size, num_kv_heads, fd), dtype=dt, device=device)
    raise ValueError(layout)


def kv_dtype_of(pool: torch.Tensor) -> int:
    if pool.dtype not in _KV_OF_TORCH:
        raise ValueError(f"pool dtype {pool.dtype} is not a cache format (uint8, float8_e4m3fn, float8_e5m2)")
    return _KV_OF_TORCH[pool.dtype]


def _desc(pool: torch.Tensor) -> CacheDesc:
    """The C descriptor of a pool view (checked for shape, not for device)."""
    if not isinstance(pool, torch.Tensor):
        raise ValueError("pool must be a torch tensor")
    kv = kv_dtype_of(pool)
    if pool.dim() != 5 or pool.shape[1] != 2 or pool.stride(4) != 1:
        raise ValueError("pool must be a (num_blocks, 2, block_size, num_kv_heads, row) view "
                         "with a contiguous last axis")
    nb, _, bs, hkv, fd = pool.shape
    if kv == KV_NVFP4:
        D = fd * 16 // 9
        if D // 2 + D // 16 != fd:
            raise ValueError(f"last axis {fd} is not a packed NVFP4 row width")
    else:
        D = fd
    st = pool.stride()
    return CacheDesc(pool.data_ptr(), nb, bs, hkv, D, kv, st[0], st[1], st[2], st[3])


def append(pool, key, value, slot_mapping, k_scale, v_scale) -> None:
    """Quantise bf16 key/value [N, Hkv, D] into the pool at slot_mapping (int64 [>= N])."""
    d = _desc(pool)
    _meta(key, "key", torch.bfloat16)
    _meta(value, "value", torch.bfloat16)
    _meta(slot_mapping, "slot_mapping", torch.int64)
    _scalar(k_scale, "k_scale")
    _scalar(v_scale, "v_scale")
    _shape(key, "key", (None, d.num_kv_heads, d.head_size))
    n = key.shape[0]
    _shape(value, "value", (n, d.num_kv_heads, d.head_size))
    if slot_mapping.dim() != 1 or slot_mapping.numel() < n:
        raise ValueError(f"slot_mapping must be 1-D with at least {n} entries, got {tuple(slot_mapping.shape)}")
    if key.stride(-1) != 1 or value.stride(-1) != 1 or not slot_mapping.is_contiguous():
        raise ValueError("key/value need a contiguous last axis and slot_mapping must be contiguous")
    _devices((pool, "pool"), (key, "key"), (value, "value"), (slot_mapping, "slot_mapping"),
             (k_scale, "k_scale"), (v_scale, "v_scale"))
    _check(library().nvfp4_kv_append(ctypes.byref(d), _ptr(key), key.stride(0), key.stride(1), _ptr(value),
                                      value.stride(0), value.stride(1), _ptr(slot_mapping), n, _ptr(k_scale),
                                      _ptr(v_scale), _stream()))


def dequant_paged(pool, block_table, seq_lens, cu_seqlens_out, max_seq_len, k_scale, v_scale,
                  out_key, out_value) -> None:
    """Gather every sequence's cache as bf16 rows [sum(seq_lens), Hkv, D]."""
    d = _desc(pool)
    for t, nm, dt in ((block_table, "block_table", torch.int32), (seq_lens, "seq_lens", torch.int32),
                      (cu_seqlens_out, "cu_seqlens_out", torch.int32), (out_key, "out_key", torch.bfloat16),
                      (out_value, "out_value", torch.bfloat16)):
        _meta(t, nm, dt)
    _scalar(k_scale, "k_scale")
    _scalar(v_scale, "v_scale")
    B = seq_lens.numel()
    _shape(seq_lens, "seq_lens", (B,))
    _shape(cu_seqlens_out, "cu_seqlens_out", (B,))
    if block_table.dim() != 2 or block_table.shape[0] < B or block_table.shape[1] < 1:
        raise ValueError(f"block_table must be [>= {B}, >= 1], got {tuple(block_table.shape)}")
    _shape(out_key, "out_key", (None, d.num_kv_heads, d.head_size))
    _shape(out_value, "out_value", tuple(out_key.shape))
    for t, nm in ((block_table, "block_table"), (seq_lens, "seq_lens"), (cu_seqlens_out, "cu_seqlens_out"),
                  (out_key, "out_key"), (out_value, "out_value")):
        if not t.is_contiguous():
            raise ValueError(f"{nm} must be contiguous")
    _devices((pool, "pool"), (block_table, "block_table"), (seq_lens, "seq_lens"),
             (cu_seqlens_out, "cu_seqlens_out"), (out_key, "out_key"), (out_value, "out_value"),
             (k_scale, "k_scale"), (v_scale, "v_scale"))
    _check(library().nvfp4_kv_dequant_paged(ctypes.byref(d), _ptr(block_table), block_table.shape[1],
                                             _ptr(seq_lens), _ptr(cu_seqlens_out), B,
                                             int(max_seq_len), _ptr(k_scale), _ptr(v_scale), _ptr(out_key),
                                             _ptr(out_value), out_key.shape[0], _stream()))


def dequant_pages(pool, page_ids, k_scale, v_scale, out) -> None:
    """Page-form dequantize: listed pages of the quantised pool (logical view)
    into the bf16 pages of ``out``, a tensor of logical shape (num_blocks, 2,
    block_size, num_kv_heads, head_size) with any strides (multiples of 8
    elements, last axis contiguous). ``page_ids`` int32 (None: pages
    0 .. num_blocks - 1)."""
    d = _desc(pool)
    _meta(out, "out", torch.bfloat16)
    _scalar(k_scale, "k_scale")
    _scalar(v_scale, "v_scale")
    if page_ids is not None:
        _meta(page_ids, "page_ids", torch.int32)
        if page_ids.dim() != 1 or not page_ids.is_contiguous():
            raise ValueError("page_ids must be 1-D and contiguous")
    _shape(out, "out", (d.num_blocks, 2, d.block_size, d.num_kv_heads, d.head_size))
    if out.stride(4) != 1:
        raise ValueError("out needs a contiguous last axis")
    _devices((pool, "pool"), (out, "out"), (page_ids, "page_ids"), (k_scale, "k_scale"), (v_scale, "v_scale"))
    n = page_ids.numel() if page_ids is not None else d.num_blocks
    st = out.stride()
    _check(library().nvfp4_kv_dequant_pages(ctypes.byref(d), _ptr(page_ids), n, _ptr(k_scale), _ptr(v_scale),
                                             _ptr(out), st[0], st[1], st[2], st[3], _stream()))


def qdq(key, value, k_scale, v_scale) -> None:
    """Quantize-dequantize emulation, in place: key, value bf16 [T, Hkv, D]."""
    _meta(key, "key", torch.bfloat16)
    _meta(value, "value", torch.bfloat16)
    _scalar(k_scale, "k_scale")
    _scalar(v_scale, "v_scale")
    if key.dim() != 3:
        raise ValueError(f"key must be [T, Hkv, D], got {tuple(key.shape)}")
    _shape(value, "value", tuple(key.shape))
    if key.stride(2) != 1 or value.stride(2) != 1:
        raise ValueError("key and value need a contiguous last axis")
    _devices((key, "key"), (value, "value"), (k_scale, "k_scale"), (v_scale, "v_scale"))
    T, H, D = key.shape
    _check(library().nvfp4_kv_qdq(_ptr(key), key.stride(0), key.stride(1), _ptr(value), value.stride(0),
                                   value.stride(1), T, H, D, _ptr(k_scale), _ptr(v_scale), _stream()))


def decode_workspace_size(num_seqs: int, num_q_heads: int, num_kv_heads: int, head_size: int) -> int:
    return int(library().nvfp4_paged_attention_decode_workspace_size(num_seqs, num_q_heads, num_kv_heads,
                                                                      head_size))


def prefill_workspace_size(head_size: int) -> int:
    """Bytes of the key-split prefill's workspace on the current device (0 for a head size not built)."""
    return int(library().nvfp4_paged_attention_prefill_workspace_size(head_size))


DECODE_SPLIT_K, DECODE_PER_PAIR = 0, 1


def decode_plan(num_seqs: int, num_kv_heads: int, head_size: int, block_size: int, max_blocks_per_seq: int,
                max_seq_len: int, kv_dtype: str = "nvfp4") -> int:
    """Which decode kernel a call with these sizes launches on the current
    device: DECODE_PER_PAIR, DECODE_SPLIT_K, or -1 for an unsupported head size."""
    return int(library().nvfp4_paged_attention_decode_plan(num_seqs, num_kv_heads, head_size, block_size,
                                                            max_blocks_per_seq, max_seq_len,
                                                            KV_DTYPES[kv_dtype][0]))


def _check_attention_args(d, q, out, block_table, seq_lens, o_scale, k_scale, v_scale):
    """Shared checks of decode and prefill: q [T, Hq, D] with Hq a multiple
    of the pool's kv heads, out of q's shape (bf16, or uint8 FP8 codes with an
    output scale), a block table row for every sequence."""
    _meta(q, "q", torch.bfloat16)
    _meta(out, "out", torch.bfloat16 if o_scale is None else torch.uint8)
    _meta(block_table, "block_table", torch.int32)
    _meta(seq_lens, "seq_lens", torch.int32)
    _scalar(k_scale, "k_scale")
    _scalar(v_scale, "v_scale")
    if o_scale is not None:
        _scalar(o_scale, "o_scale")
    if q.dim() != 3 or q.shape[2] != d.head_size or q.shape[1] < 1 or q.shape[1] % d.num_kv_heads != 0:
        raise ValueError(f"q must be [tokens, Hq, {d.head_size}] with Hq a multiple of {d.num_kv_heads}, "
                         f"got {tuple(q.shape)}")
    _shape(out, "out", tuple(q.shape))
    B = seq_lens.numel()
    _shape(seq_lens, "seq_lens", (B,))
    if block_table.dim() != 2 or block_table.shape[0] < B or block_table.shape[1] < 1:
        raise ValueError(f"block_table must be [>= {B}, >= 1], got {tuple(block_table.shape)}")
    for t, nm in ((block_table, "block_table"), (seq_lens, "seq_lens"), (out, "out")):
        if not t.is_contiguous():
            raise ValueError(f"{nm} must be contiguous")
    if q.stride(-1) != 1:
        raise ValueError("q needs a contiguous last axis")
    return B


def paged_attention_decode(pool, q, block_table, seq_lens, max_seq_len, k_scale, v_scale, sm_scale,
                           out, workspace, o_scale=None) -> None:
    """One query token per sequence: q bf16 [B, Hq, D]; workspace uint8. out is
    bf16 [B, Hq, D], or, with an output scale ``o_scale`` (device fp32
    scalar), uint8 [B, Hq, D] of FP8-E4M3 codes (see fp8_to_bf16)."""
    d = _desc(pool)
    B = _check_attention_args(d, q, out, block_table, seq_lens, o_scale, k_scale, v_scale)
    if q.shape[0] != B:
        raise ValueError(f"q must have one row per sequence ({B}), got {q.shape[0]}")
    _meta(workspace, "workspace", torch.uint8)
    if not workspace.is_contiguous():
        raise ValueError("workspace must be contiguous")
    _devices((pool, "pool"), (q, "q"), (out, "out"), (block_table, "block_table"), (seq_lens, "seq_lens"),
             (workspace, "workspace"), (k_scale, "k_scale"), (v_scale, "v_scale"), (o_scale, "o_scale"))
    args = (ctypes.byref(d), _ptr(q), q.stride(0), q.stride(1), q.shape[1], _ptr(block_table), block_table.shape[1],
            _ptr(seq_lens), B, int(max_seq_len), _ptr(k_scale), _ptr(v_scale), float(sm_scale))
    if o_scale is None:
        _check(library().nvfp4_paged_attention_decode(*args, _ptr(out), _ptr(workspace),
                                                      workspace.numel(), _stream()))
    else:
        _check(library().nvfp4_paged_attention_decode_fp8(*args, _ptr(o_scale), _ptr(out), _ptr(workspace),
                                                          workspace.numel(), _stream()))


def paged_attention_decode_noalloc(pool, q, block_table, seq_lens, max_seq_len, k_scale, v_scale, sm_scale,
                                   out) -> None:
    """paged_attention_decode without a workspace: the split-K scratch is the
    library's own fixed device array (32 MiB per GPU), so the call allocates
    nothing. Calls that overlap on one GPU race on that array."""
    d = _desc(pool)
    B = _check_attention_args(d, q, out, block_table, seq_lens, None, k_scale, v_scale)
    if q.shape[0] != B:
        raise ValueError(f"q must have one row per sequence ({B}), got {q.shape[0]}")
    _devices((pool, "pool"), (q, "q"), (out, "out"), (block_table, "block_table"), (seq_lens, "seq_lens"),
             (k_scale, "k_scale"), (v_scale, "v_scale"))
    _check(library().nvfp4_paged_attention_decode_noalloc(
        ctypes.byref(d), _ptr(q), q.stride(0), q.stride(1), q.shape[1], _ptr(block_table), block_table.shape[1],
        _ptr(seq_lens), B, int(max_seq_len), _ptr(k_scale), _ptr(v_scale), float(sm_scale), _ptr(out), _stream()))


def fp8_to_bf16(codes, o_scale, out) -> None:
    """The FP8 output's epilogue: uint8 codes -> bf16 of the same shape."""
    _meta(codes, "codes", torch.uint8)
    _meta(out, "out", torch.bfloat16)
    _scalar(o_scale, "o_scale")
    _shape(out, "out", tuple(codes.shape))
    if not codes.is_contiguous() or not out.is_contiguous():
        raise ValueError("codes and out must be contiguous")
    _devices((codes, "codes"), (out, "out"), (o_scale, "o_scale"))
    _check(library().nvfp4_fp8_to_bf16(_ptr(codes), codes.numel(), _ptr(o_scale), _ptr(out), _stream()))


def quant_activations_scale_bytes(m: int, k: int, swizzled: bool = True) -> int:
    return int(library().nvfp4_quant_activations_scale_bytes(int(m), int(k), 1 if swizzled else 0))


def quant_activations(x, global_scale, swizzled: bool = True, codes=None, scales=None):
    """bf16 [m, k] -> (codes uint8 [m, k/2], scales uint8): the scales are
    [m, k/16] row-major, or the flat swizzled 128 x 4 tile buffer."""
    _meta(x, "x", torch.bfloat16)
    _scalar(global_scale, "global_scale")
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be 2-D with a contiguous last axis")
    m, k = x.shape
    nbytes = quant_activations_scale_bytes(m, k, swizzled)
    if nbytes < 0:
        raise ValueError("k must be a positive multiple of 16")
    if codes is not None:
        _meta(codes, "codes", torch.uint8)
        _shape(codes, "codes", (m, k // 2))
        if not codes.is_contiguous():
            raise ValueError("codes must be contiguous")
    if scales is not None:
        _meta(scales, "scales", torch.uint8)
        if scales.numel() != nbytes or not scales.is_contiguous():
            raise ValueError(f"scales must be contiguous with {nbytes} bytes")
    _devices((x, "x"), (global_scale, "global_scale"), (codes, "codes"), (scales, "scales"))
    if codes is None:
        codes = torch.empty((m, k // 2), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty(nbytes if swizzled else (m, k // 16), dtype=torch.uint8, device=x.device)
    _check(library().nvfp4_quant_activations(_ptr(x), x.stride(0), m, k, _ptr(global_scale), 1 if swizzled else 0,
                                             _ptr(codes), _ptr(scales), _stream()))
    return codes, scales


def paged_attention_prefill(pool, q, cu_seqlens_q, max_q_len, block_table, seq_lens, max_seq_len,
                            k_scale, v_scale, sm_scale, out, causal: bool = True, o_scale=None,
                            workspace=None) -> None:
    """Chunked prefill: q bf16 [total_q, Hq, D]; cu_seqlens_q int32 [B + 1]. out is
    bf16 [total_q, Hq, D], or with an output scale ``o_scale`` uint8 FP8-E4M3 codes.
    ``workspace`` (uint8, zero-filled once, at least ``prefill_workspace_size(D)``
    bytes) selects the key split: every workgroup takes an equal share of the steps."""
    d = _desc(pool)
    B = _check_attention_args(d, q, out, block_table, seq_lens, o_scale, k_scale, v_scale)
    _meta(cu_seqlens_q, "cu_seqlens_q", torch.int32)
    _shape(cu_seqlens_q, "cu_seqlens_q", (B + 1,))
    if not cu_seqlens_q.is_contiguous():
        raise ValueError("cu_seqlens_q must be contiguous")
    ws_ptr, ws_bytes = ctypes.c_void_p(0), 0
    if workspace is not None:
        _meta(workspace, "workspace", torch.uint8)
        if not workspace.is_contiguous():
            raise ValueError("workspace must be contiguous")
        ws_ptr, ws_bytes = _ptr(workspace), workspace.numel()
    _devices((pool, "pool"), (q, "q"), (out, "out"), (block_table, "block_table"), (seq_lens, "seq_lens"),
             (cu_seqlens_q, "cu_seqlens_q"), (k_scale, "k_scale"), (v_scale, "v_scale"), (o_scale, "o_scale"),
             (workspace, "workspace"))
    common = (ctypes.byref(d), _ptr(q), q.stride(0), q.stride(1), q.shape[1], _ptr(cu_seqlens_q), int(max_q_len),
              q.shape[0], _ptr(block_table), block_table.shape[1], _ptr(seq_lens), B,
              int(max_seq_len), _ptr(k_scale), _ptr(v_scale), float(sm_scale), 1 if causal else 0)
    if o_scale is None:
        _check(library().nvfp4_paged_attention_prefill(*common, _ptr(out), ws_ptr, ws_bytes, _stream()))
    else:
        _check(library().nvfp4_paged_attention_prefill_fp8(*common, _ptr(o_scale), _ptr(out), ws_ptr, ws_bytes,
                                                           _stream()))
