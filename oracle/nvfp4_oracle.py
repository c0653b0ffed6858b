"""CPU oracle for the NVFP4-quantised paged KV cache.

TEST INFRASTRUCTURE ONLY. Nothing in the library imports this module; only the
tests, the smoke check and the benchmark's CPU-baseline leg may call it. It
shares no code, table or constant generator with the HIP path.

What it computes, and where each step comes from (sources are the three pages
the method is described on):

* [P40177] "FlashInfer backend adds end-to-end NVFP4 KV cache support" (vLLM PR
  40177 summary): the pool shape and packed width in the ``get_kv_cache_shape``
  snippet; "uint8 holding packed FP4 data and the FP8 block scale" in the
  ``get_dtype_for_flashinfer`` snippet; the slot-mapping writer and the HND
  view in the ``_create_nvfp4_hnd_kv_cache`` test snippet.
* [P39129] "Move NVFP4 GEMM management into NvFp4LinearKernel" (vLLM PR 39129
  report): the ``NvFp4LinearLayerConfig`` docstring fixes the format itself —
  two FP4 values per byte, one FP8-E4M3 scale per group of 16, plus global
  fp32 scale scalars.
* [RFC47684] "[RFC]: FlashInfer NVFP4 KV serving on pre-SM100 GPUs": the
  quantise-append-with-slot-mapping writer and the paged dequantize used on the
  fallback read path ("Cause analysis", "Fix steps").

The pages print neither the bit order inside a byte nor the quantiser's
arithmetic. The readings taken here (each listed in the design notes):
E2M1 codes are OCP sign|e1e0|m; element 2k sits in the low nibble of byte k;
the D/2 data bytes precede the D/16 scale bytes; the kv scale ``g`` is a
dequantisation multiplier; the block scale is RNE-to-E4M3 of amax/(6g),
saturating at 448; elements are multiplied by the fp32 reciprocal of the
block step and rounded to E2M1 with ties to even, saturating at 6; slots
outside the pool are skipped. Quantiser arithmetic is IEEE fp32 with
round-to-nearest-even (NumPy float32 operations), attention is fp64.
"""
from __future__ import annotations

import numpy as np

F32 = np.float32

# ---------------------------------------------------------------------------
# Layout  [P40177, "Key source snippets", get_kv_cache_shape]
# ---------------------------------------------------------------------------


def full_dim(head_size: int) -> int:
    """Bytes per (token, head) row: head_size/2 packed FP4 bytes plus one FP8
    scale per 16 elements."""
    assert head_size % 16 == 0
    return head_size // 2 + head_size // 16


# Cache dtypes [P40177 "Key source snippets": the backend's supported KV cache
# dtypes list fp8 / fp8_e4m3 / fp8_e5m2 beside nvfp4; get_dtype_for_flashinfer
# maps them to float8_e4m3fn, float8_e5m2 and uint8]. An FP8 row is head_size
# bytes, one code per element, under the per-tensor scale alone.
KV_DTYPES = ("nvfp4", "fp8_e4m3", "fp8_e5m2")


def row_bytes(head_size: int, kv_dtype: str = "nvfp4") -> int:
    assert kv_dtype in KV_DTYPES
    return full_dim(head_size) if kv_dtype == "nvfp4" else head_size


def pool_shape(num_blocks: int, block_size: int, num_kv_heads: int, head_size: int, kv_dtype: str = "nvfp4"):
    """Logical pool shape (num_blocks, 2, block_size, num_kv_heads, row bytes)."""
    return (num_blocks, 2, block_size, num_kv_heads, row_bytes(head_size, kv_dtype))


# ---------------------------------------------------------------------------
# bf16 (inputs and the standalone dequant's output)
# ---------------------------------------------------------------------------


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> fp32 (exact: bf16 is the top half of fp32)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(F32)


def f32_to_bf16(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest, ties to even (finite x)."""
    u = np.ascontiguousarray(x, dtype=F32).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    return ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint16)


# ---------------------------------------------------------------------------
# FP8 E4M3 block scale  [P39129, nvfp4/base.py snippet, NvFp4LinearLayerConfig]
# OCP E4M3FN: 1 sign, 4 exponent bits (bias 7), 3 mantissa bits, no infinity,
# 0x7F / 0xFF are NaN, largest finite 448 (0x7E).
# ---------------------------------------------------------------------------


def e4m3_decode(b: np.ndarray) -> np.ndarray:
    """E4M3FN byte -> value (float64; NaN for 0x7F/0xFF)."""
    b = np.asarray(b, dtype=np.int64)
    sign = np.where(b >> 7, -1.0, 1.0)
    e = (b >> 3) & 15
    m = b & 7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((b & 0x7F) == 0x7F, np.nan, mag)
    return sign * mag


def e4m3_encode_sat(s: np.ndarray) -> np.ndarray:
    """Non-negative fp32 -> E4M3FN byte, round to nearest, ties to even,
    saturating to 448 (0x7E) instead of producing NaN; +inf (an overflowed
    amax / (6 g)) saturates too.

    Within the binade [2^e, 2^(e+1)) (e >= -6; below that the subnormal step
    2^-9 continues) the step is 2^(e-3); n = rint(s / step) is the significand
    count and the byte is (e + 6) * 8 + n, which also carries a round-up into
    the next binade (n = 16) and the subnormal/normal boundary correctly.
    """
    s = np.asarray(s, dtype=np.float64)  # fp32 values are exact in fp64
    assert np.all(s >= 0)                # also rejects NaN
    s = np.minimum(s, 448.0)             # everything from 448 up, +inf included, saturates
    pos = s > 0
    e = np.floor(np.log2(np.where(pos, s, 1.0)))
    # guard log2 rounding near powers of two
    e = np.where(pos & (np.exp2(e) > s), e - 1, e)
    e = np.where(pos & (np.exp2(e + 1) <= s), e + 1, e)
    # zero (and everything below the normal range) uses the subnormal step
    e = np.where(pos, np.maximum(e, -6.0), -6.0)
    n = np.rint(s / np.exp2(e - 3.0))  # numpy rint: ties to even
    code = (e + 6.0) * 8.0 + n
    code = np.where(s >= 448.0, 0x7E, code)
    return code.astype(np.uint8)


# OCP E5M2: 1 sign, 5 exponent bits (bias 15), 2 mantissa bits, infinities
# (0x7C, 0xFC) and NaNs (exponent 31, mantissa != 0); largest finite 57344
# (0x7B); smallest subnormal 2^-16.


def e5m2_decode(b: np.ndarray) -> np.ndarray:
    """E5M2 byte -> value (float64; +-inf and NaN where the format has them)."""
    b = np.asarray(b, dtype=np.int64)
    sign = np.where(b >> 7, -1.0, 1.0)
    e = (b >> 2) & 31
    m = b & 3
    mag = np.where(e == 0, m * 2.0 ** -16, (1.0 + m / 4.0) * np.exp2(e - 15.0))
    mag = np.where(e == 31, np.where(m == 0, np.inf, np.nan), mag)
    return sign * mag


def _fp8_encode_mag(a: np.ndarray, mbits: int, emin: int, maxv: float, maxcode: int) -> np.ndarray:
    """Non-negative magnitudes -> FP8 magnitude codes (RNE, saturating to the
    largest finite value): in binade [2^e, 2^(e+1)), e clamped to >= emin
    (the subnormal step continues below), the significand count is
    n = rint(a / 2^(e - mbits)) and the code is (e - emin) * 2^mbits + n."""
    a = np.minimum(np.asarray(a, dtype=np.float64), maxv)
    pos = a > 0
    e = np.floor(np.log2(np.where(pos, a, 1.0)))
    e = np.where(pos & (np.exp2(e) > a), e - 1, e)
    e = np.where(pos & (np.exp2(e + 1) <= a), e + 1, e)
    e = np.where(pos, np.maximum(e, float(emin)), float(emin))
    n = np.rint(a / np.exp2(e - mbits))
    code = (e - emin) * 2.0 ** mbits + n
    return np.minimum(code, maxcode).astype(np.uint8)


def fp8_encode(x: np.ndarray, kind: str) -> np.ndarray:
    """fp32 -> FP8 byte ("e4m3": E4M3FN, "e5m2"), round to nearest, ties to
    even, magnitudes from the largest finite value up (infinity included)
    saturate to it; the sign bit is copied from x (-0 -> 0x80). NaN is outside
    the contract."""
    x = np.asarray(x, dtype=F32)
    assert not np.any(np.isnan(x))
    if kind == "e4m3":
        mag = _fp8_encode_mag(np.abs(x), 3, -6, 448.0, 0x7E)
    elif kind == "e5m2":
        mag = _fp8_encode_mag(np.abs(x), 2, -14, 57344.0, 0x7B)
    else:
        raise ValueError(kind)
    sign = (x.view(np.uint32) >> np.uint32(31)).astype(np.uint8)
    return (sign << np.uint8(7)) | mag


def fp8_decode(b: np.ndarray, kind: str) -> np.ndarray:
    return e4m3_decode(b) if kind == "e4m3" else e5m2_decode(b)


# ---------------------------------------------------------------------------
# FP4 E2M1 element  [P39129 NvFp4LinearLayerConfig: "two FP4 values per byte";
# P40177 get_dtype_for_flashinfer: packed FP4 data in uint8]
# OCP E2M1: 1 sign, 2 exponent bits (bias 1), 1 mantissa bit.
# ---------------------------------------------------------------------------

E2M1_MAGNITUDES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def e2m1_decode(code: np.ndarray) -> np.ndarray:
    code = np.asarray(code, dtype=np.int64)
    mag = E2M1_MAGNITUDES[code & 7]
    return np.where(code & 8, -mag, mag)


def e2m1_encode(v: np.ndarray) -> np.ndarray:
    """fp32 -> 4-bit code, round to nearest with ties to the even code
    (mantissa bit 0), |v| above 6 saturating to 6. The sign bit is copied from
    v, so -0 encodes as 0x8.

    Midpoints between neighbouring magnitudes and where their ties go:
    0.25 -> 0, 0.75 -> 1, 1.25 -> 1, 1.75 -> 2, 2.5 -> 2, 3.5 -> 4, 5 -> 4.
    """
    v = np.asarray(v, dtype=F32)
    a = np.abs(v)
    idx = ((a > F32(0.25)).astype(np.uint8) + (a >= F32(0.75)) + (a > F32(1.25))
           + (a >= F32(1.75)) + (a > F32(2.5)) + (a >= F32(3.5)) + (a > F32(5.0)))
    sign = (v.view(np.uint32) >> np.uint32(31)).astype(np.uint8)
    return (sign << np.uint8(3)) | idx.astype(np.uint8)


# ---------------------------------------------------------------------------
# Row quantiser: the slot-mapping writer's arithmetic
# [P40177 "_create_nvfp4_hnd_kv_cache": bf16 tokens [N, H, D] quantised into
#  the uint8 pool through reshape_and_cache_flash(..., "nvfp4", kv_scale,
#  kv_scale); RFC47684 "Cause analysis": quantize-append with slot mapping]
# ---------------------------------------------------------------------------


def quantize_rows(x_bits: np.ndarray, g) -> np.ndarray:
    """bf16 rows [..., D] -> packed rows [..., D/2 + D/16] (uint8).

    Per 16-element block: amax -> s = E4M3(amax / (6 g)); step d = s * g;
    r = 1 / d (0 when d == 0); code_i = E2M1(x_i * r). Every operation is one
    fp32 RNE operation, in this order.
    """
    x = bf16_to_f32(x_bits)
    D = x.shape[-1]
    lead = x.shape[:-1]
    g = F32(g)
    blk = x.reshape(lead + (D // 16, 16))
    amax = np.max(np.abs(blk), axis=-1)                       # exact
    t = F32(6.0) * g
    with np.errstate(over="ignore"):  # an overflowed quotient saturates below
        s32 = (amax / t).astype(F32)
    s8 = e4m3_encode_sat(s32)
    d = (e4m3_decode(s8).astype(F32) * g).astype(F32)
    with np.errstate(divide="ignore"):
        r = np.where(d == 0, F32(0.0), F32(1.0) / d).astype(F32)
    with np.errstate(over="ignore"):  # overflowed products saturate to +-6 below
        v = (blk * r[..., None]).astype(F32)
    codes = e2m1_encode(v).reshape(lead + (D,))
    data = (codes[..., 0::2] | (codes[..., 1::2] << np.uint8(4))).astype(np.uint8)
    return np.concatenate([data, s8], axis=-1)


def quantize_rows_fp8(x_bits: np.ndarray, g, kind: str) -> np.ndarray:
    """bf16 rows [..., D] -> FP8 rows [..., D] (uint8) under the per-tensor
    scale g: code = FP8(RN32(x / g)), one fp32 division per element."""
    x = bf16_to_f32(x_bits)
    with np.errstate(over="ignore"):  # an overflowed quotient saturates
        q = (x / F32(g)).astype(F32)
    return fp8_encode(q, kind)


def dequantize_rows_fp8(rows: np.ndarray, g, kind: str) -> np.ndarray:
    """FP8 rows [..., D] -> fp32 values RN32(fp8 * g)."""
    return (fp8_decode(rows, kind).astype(F32) * F32(g)).astype(F32)


def quantize_kv(x_bits: np.ndarray, g, kv_dtype: str = "nvfp4") -> np.ndarray:
    """Rows as the cache of kv_dtype stores them."""
    if kv_dtype == "nvfp4":
        return quantize_rows(x_bits, g)
    return quantize_rows_fp8(x_bits, g, kv_dtype[4:])


def dequantize_kv(rows: np.ndarray, g, head_size: int, kv_dtype: str = "nvfp4") -> np.ndarray:
    """Stored rows of a cache of kv_dtype -> fp32 values."""
    if kv_dtype == "nvfp4":
        return dequantize_rows(rows, g, head_size)
    return dequantize_rows_fp8(rows, g, kv_dtype[4:])


def dequantize_rows(rows: np.ndarray, g, head_size: int) -> np.ndarray:
    """Packed rows [..., full_dim] -> fp32 values [..., D]:
    x = fp32( (E2M1(code) * E4M3(scale)) * g ); the inner product is exact."""
    D = head_size
    rows = np.asarray(rows, dtype=np.uint8)
    data = rows[..., : D // 2]
    scales = rows[..., D // 2: D // 2 + D // 16]
    codes = np.empty(rows.shape[:-1] + (D,), np.uint8)
    codes[..., 0::2] = data & np.uint8(15)
    codes[..., 1::2] = data >> np.uint8(4)
    cs = e2m1_decode(codes) * np.repeat(e4m3_decode(scales), 16, axis=-1)
    return (cs.astype(F32) * F32(g)).astype(F32)


def append(pool: np.ndarray, key_bits: np.ndarray, value_bits: np.ndarray,
           slot_mapping: np.ndarray, k_scale, v_scale, kv_dtype: str = "nvfp4") -> np.ndarray:
    """Slot-mapping writer on a logical pool (num_blocks, 2, bs, Hkv, fd).

    Token t goes to block slot // bs, row slot % bs; K at index 0 and V at 1
    of the second axis [P40177 get_kv_cache_shape]. Slots below 0 or past the
    pool are skipped. Modifies and returns ``pool``.
    """
    nb, two, bs, hkv, fd = pool.shape
    slots = np.asarray(slot_mapping, dtype=np.int64)
    ok = (slots >= 0) & (slots < nb * bs)
    slots = slots[ok]
    if slots.size == 0:
        return pool
    kq = quantize_kv(np.asarray(key_bits)[ok], k_scale, kv_dtype)
    vq = quantize_kv(np.asarray(value_bits)[ok], v_scale, kv_dtype)
    pool[slots // bs, 0, slots % bs] = kq
    pool[slots // bs, 1, slots % bs] = vq
    return pool


def gather_rows(pool: np.ndarray, block_table_row: np.ndarray, length: int, kv: int) -> np.ndarray:
    """Packed rows of tokens 0..length-1 of one sequence: token j lives in
    block block_table_row[j // bs], row j % bs."""
    bs = pool.shape[2]
    j = np.arange(length)
    return pool[np.asarray(block_table_row, np.int64)[j // bs], kv, j % bs]


def dequant_paged(pool: np.ndarray, block_table: np.ndarray, seq_lens: np.ndarray,
                  k_scale, v_scale, head_size: int, kv_dtype: str = "nvfp4"):
    """Paged dequantize [RFC47684 "Fix steps": nvfp4_kv_dequantize_paged]:
    every sequence's keys and values gathered through the block table and
    written, one sequence after another, as bf16 [sum(seq_lens), Hkv, D]."""
    ks, vs = [], []
    for b in range(len(seq_lens)):
        L = int(seq_lens[b])
        ks.append(f32_to_bf16(dequantize_kv(gather_rows(pool, block_table[b], L, 0), k_scale, head_size, kv_dtype)))
        vs.append(f32_to_bf16(dequantize_kv(gather_rows(pool, block_table[b], L, 1), v_scale, head_size, kv_dtype)))
    hkv = pool.shape[3]
    empty = np.zeros((0, hkv, head_size), np.uint16)
    return (np.concatenate(ks) if ks else empty, np.concatenate(vs) if vs else empty)


# ---------------------------------------------------------------------------
# The codec on its own, for paths without native FP4 attention
# [P40177 "Related context": the NVFP4 dequantization and quantize-dequantize
#  (QDQ) emulation kernels for Hopper / AMD Instinct; RFC47684 "Fix steps":
#  nvfp4_kv_dequantize_paged]
# ---------------------------------------------------------------------------


def dequant_pages(pool: np.ndarray, page_ids, k_scale, v_scale, head_size: int, kv_dtype: str = "nvfp4") -> np.ndarray:
    """Page-form dequantize: every listed page of the logical pool (num_blocks,
    2, bs, Hkv, full_dim) becomes a bf16 page (2, bs, Hkv, D) whose rows are
    dequantize_rows of the packed rows, rounded to bf16, so that one block
    table addresses both caches. Returns [len(page_ids), 2, bs, Hkv, D] bf16
    bits in the order given."""
    ids = np.asarray(page_ids, dtype=np.int64)
    pages = pool[ids]                                       # [P, 2, bs, Hkv, fd]
    k = f32_to_bf16(dequantize_kv(pages[:, 0], k_scale, head_size, kv_dtype))
    v = f32_to_bf16(dequantize_kv(pages[:, 1], v_scale, head_size, kv_dtype))
    return np.stack([k, v], axis=1)


def qdq_rows(x_bits: np.ndarray, g, head_size: int) -> np.ndarray:
    """Quantize-dequantize emulation of bf16 rows [..., D]: the rows are
    quantised as the append writes them and read back as the dequantize
    returns them (bf16 bits)."""
    return f32_to_bf16(dequantize_rows(quantize_rows(x_bits, g), g, head_size))


# ---------------------------------------------------------------------------
# Paged attention over the quantised cache (decode and chunked prefill)
# [P40177 "Implementation breakdown" items 1 and 3: prefill/decode wrappers
#  reading the packed cache plus its block-scale view; RFC47684 "Cause
#  analysis": attention on the paged read path]
# ---------------------------------------------------------------------------


def paged_attention(pool: np.ndarray, query_bits: np.ndarray, cu_q: np.ndarray,
                    block_table: np.ndarray, seq_lens: np.ndarray, k_scale, v_scale,
                    sm_scale, head_size: int, causal: bool = True, kv_dtype: str = "nvfp4") -> np.ndarray:
    """Softmax attention of each sequence's queries over all of its cached keys.

    Sequence b has L = seq_lens[b] keys and q = cu_q[b+1] - cu_q[b] queries,
    the last q of its L tokens; query i sees keys j <= L - q + i when causal,
    all L keys otherwise. q head h reads kv head h // (Hq / Hkv). Scores are
    (q . K^) * sm_scale with K^, V^ the fp32 dequantised cache; everything
    after dequantisation is fp64. Returns fp64 [sum(q), Hq, D]; rows with no
    visible key are 0.
    """
    q_all = bf16_to_f32(query_bits).astype(np.float64)
    T, Hq, D = q_all.shape
    Hkv = pool.shape[3]
    G = Hq // Hkv
    out = np.zeros((T, Hq, D), np.float64)
    sm = float(F32(sm_scale))
    for b in range(len(seq_lens)):
        L = int(seq_lens[b])
        q0, q1 = int(cu_q[b]), int(cu_q[b + 1])
        nq = q1 - q0
        if nq == 0 or L == 0:
            continue
        K = dequantize_kv(gather_rows(pool, block_table[b], L, 0), k_scale, D, kv_dtype).astype(np.float64)
        V = dequantize_kv(gather_rows(pool, block_table[b], L, 1), v_scale, D, kv_dtype).astype(np.float64)
        if causal:
            limit = L - nq + np.arange(nq)               # last visible key per query
            visible = np.arange(L)[None, :] <= limit[:, None]
        else:
            visible = np.ones((nq, L), bool)
        for h in range(Hq):
            kvh = h // G
            s = (q_all[q0:q1, h, :] @ K[:, kvh, :].T) * sm        # [nq, L]
            s = np.where(visible, s, -np.inf)
            m = np.max(s, axis=1, keepdims=True)
            has = np.isfinite(m[:, 0])
            w = np.where(visible, np.exp(s - np.where(has[:, None], m, 0.0)), 0.0)
            den = w.sum(axis=1, keepdims=True)
            o = (w @ V[:, kvh, :]) / np.where(den > 0, den, 1.0)
            out[q0:q1, h, :] = np.where(has[:, None], o, 0.0)
    return out


# ---------------------------------------------------------------------------
# FP8 attention output and its dequantize-to-bf16 epilogue [P40177
# "Implementation breakdown" item 2: the NVFP4 attention kernel emits FP8
# into a preallocated buffer and the forward pass dequantises it back to the
# model dtype; "Risks and impact": that FP8 output adds a rounding step]
# ---------------------------------------------------------------------------


def fp8_out(o: np.ndarray, o_scale) -> np.ndarray:
    """Attention output -> FP8-E4M3 codes under a per-tensor output scale:
    q = RN32(RN32(o) / o_scale) (fp32 division), then E4M3 RNE of |q|
    saturating to 448, with the sign of q in bit 7."""
    o32 = np.asarray(o).astype(F32)
    q = (o32 / F32(o_scale)).astype(F32)
    mag = e4m3_encode_sat(np.abs(q))
    sign = (q.view(np.uint32) >> np.uint32(31)).astype(np.uint8)
    return (sign << np.uint8(7)) | mag


def fp8_to_bf16(codes: np.ndarray, o_scale) -> np.ndarray:
    """The epilogue: bf16 RNE of fp32(e4m3(code) * o_scale) (bf16 bits)."""
    return f32_to_bf16((e4m3_decode(codes).astype(F32) * F32(o_scale)).astype(F32))


# ---------------------------------------------------------------------------
# Activation quantisation with swizzled block scales [P39129 "Implementation
# breakdown", the CUTLASS and FlashInfer kernels' apply_weights: the
# activation is quantised to NVFP4 under the layer's input global scale with
# is_sf_swizzled_layout=True before the FP4 GEMM; process_weights_after_loading
# rearranges block scales with swizzle_blockscale "to match the CUTLASS
# layout"]
#
# Readings: the block codec is the one quantize_rows applies, with the input
# global scale in the role of g (the inverse of the quantise-direction global
# scale is the dequantisation multiplier). The swizzled layout is the
# block-scaled GEMM operand layout of 128-row x 4-scale tiles: the scale
# matrix is zero-padded to a multiple of 128 rows and of 4 columns; tile
# (i, j) covers rows 128i..128i+127 and scale columns 4j..4j+3 and occupies
# 512 consecutive bytes, tiles in row-major order of (i, j); inside a tile,
# row 128i + 32a + b (a < 4, b < 32) puts its 4 scales at bytes 16b + 4a ..
# 16b + 4a + 3.
# ---------------------------------------------------------------------------


def sf_swizzled_shape(m: int, k: int):
    """(rows, scale columns) of the padded swizzled scale matrix."""
    nc = k // 16
    return ((m + 127) // 128) * 128, ((nc + 3) // 4) * 4


def sf_swizzle_offset(r, c, k: int):
    """Byte offset of the scale of row r, scale column c in the swizzled
    buffer of an [m, k] activation."""
    ncp = sf_swizzled_shape(0, k)[1]
    tile = (r // 128) * (ncp // 4) + c // 4
    return tile * 512 + (r % 32) * 16 + ((r % 128) // 32) * 4 + c % 4


def quant_activations(x_bits: np.ndarray, g, swizzled: bool):
    """bf16 activation [m, k] (k a multiple of 16) -> (codes [m, k/2] uint8,
    scales uint8): the scales are [m, k/16] row-major, or the flat swizzled
    buffer of size rows * cols of sf_swizzled_shape with zero padding."""
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    m, k = x_bits.shape
    packed = quantize_rows(x_bits, g)
    codes = np.ascontiguousarray(packed[:, : k // 2])
    scales = np.ascontiguousarray(packed[:, k // 2:])
    if not swizzled:
        return codes, scales
    mp, ncp = sf_swizzled_shape(m, k)
    out = np.zeros(mp * ncp, np.uint8)
    r, c = np.meshgrid(np.arange(m), np.arange(k // 16), indexing="ij")
    out[sf_swizzle_offset(r, c, k)] = scales
    return codes, out
