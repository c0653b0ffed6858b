"""Seeded workload generator (inputs only; no quantisation or attention math).

Recipe, drawn from ``numpy.random.default_rng(seed)`` in this fixed order:

1. sequence lengths (and, for mixed batches, which sequences decode),
2. the physical block permutation (10 % spare blocks unless a pool size is
   given), assigned to sequences page by page in sequence order,
3. outlier channels or per-token magnitudes,
4. K, then V, then Q: fp32 standard normal draws rounded to bf16 (RNE) by
   torch's CPU cast, one sequence at a time.

The per-tensor kv scale of the recipe is ``amax / (6 * 448)`` in fp32 over the
whole bf16 layer tensor (all tokens, including the ones appended last).

bf16 tensors are carried as ``uint16`` bit patterns so that the oracle and the
device see exactly the same bytes.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch

CONFIG_NAMES = {
    1: "tiny_decode",
    2: "small_decode",
    3: "long_decode",
    4: "chunked_prefill",
    5: "mixed_serving",
}


@dataclasses.dataclass
class Workload:
    name: str
    seed: int
    num_q_heads: int
    num_kv_heads: int
    head_size: int
    block_size: int
    num_blocks: int
    seq_lens: np.ndarray       # int32 [B]; keys per sequence after the append
    q_lens: np.ndarray         # int32 [B]; tokens appended now (queries)
    is_decode: np.ndarray      # bool  [B]
    block_table: np.ndarray    # int32 [B, max_blocks_per_seq], -1 padded
    token_offsets: np.ndarray  # int64 [B + 1]; seq b owns key/value rows [off[b], off[b+1])
    key: np.ndarray            # uint16 bf16 bits [sum(seq_lens), Hkv, D]
    value: np.ndarray          # uint16 bf16 bits [sum(seq_lens), Hkv, D]
    query: np.ndarray          # uint16 bf16 bits [sum(q_lens), Hq, D]
    cu_q: np.ndarray           # int32 [B + 1]
    slot_mapping: np.ndarray   # int64 [sum(seq_lens)]; slot of every key/value row
    k_scale: np.float32
    v_scale: np.float32

    @property
    def num_seqs(self) -> int:
        return int(self.seq_lens.shape[0])

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_table.shape[1])

    @property
    def full_dim(self) -> int:
        # pool row width in bytes, as the cache shape prescribes (D/2 + D/16)
        return self.head_size // 2 + self.head_size // 16

    def cached_mask(self) -> np.ndarray:
        """bool [sum(seq_lens)]: True for rows present before this step."""
        m = np.zeros(int(self.token_offsets[-1]), dtype=bool)
        for b in range(self.num_seqs):
            lo = int(self.token_offsets[b])
            m[lo: lo + int(self.seq_lens[b] - self.q_lens[b])] = True
        return m

    def subset(self, seqs) -> "Workload":
        """Sequences ``seqs`` only, sharing the same pool geometry and scales."""
        seqs = np.asarray(seqs, dtype=np.int64)
        rows, qrows = [], []
        for b in seqs:
            rows.append(np.arange(self.token_offsets[b], self.token_offsets[b + 1]))
            qrows.append(np.arange(self.cu_q[b], self.cu_q[b + 1]))
        rows = np.concatenate(rows) if rows else np.zeros(0, np.int64)
        qrows = np.concatenate(qrows) if qrows else np.zeros(0, np.int64)
        seq_lens = self.seq_lens[seqs]
        q_lens = self.q_lens[seqs]
        off = np.zeros(len(seqs) + 1, np.int64)
        off[1:] = np.cumsum(seq_lens)
        cu_q = np.zeros(len(seqs) + 1, np.int32)
        cu_q[1:] = np.cumsum(q_lens)
        return dataclasses.replace(
            self, seq_lens=seq_lens, q_lens=q_lens, is_decode=self.is_decode[seqs],
            block_table=self.block_table[seqs], token_offsets=off,
            key=self.key[rows], value=self.value[rows], query=self.query[qrows],
            cu_q=cu_q, slot_mapping=self.slot_mapping[rows])


def _to_bf16_bits(x: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def _bf16_bits_absmax(bits: np.ndarray) -> np.float32:
    if bits.size == 0:
        return np.float32(0.0)
    # with the sign cleared, the largest finite magnitude has the largest bit pattern
    top = np.array([np.max(bits & np.uint16(0x7FFF))], dtype=np.uint32) << np.uint32(16)
    return np.float32(top.view(np.float32)[0])


def make_workload(*, seed: int, name: str, seq_lens, q_lens, num_q_heads: int,
                  num_kv_heads: int, head_size: int, block_size: int,
                  num_blocks: int | None = None, is_decode=None,
                  k_outlier_frac: float = 0.0, k_outlier_gain: float = 1.0,
                  v_outlier_frac: float = 0.0, v_outlier_gain: float = 1.0,
                  token_lognormal_sigma: float = 0.0,
                  lengths_drawn=None, rng=None) -> Workload:
    """Build a workload from explicit lengths (the length draw, if any, is the
    caller's, made from the same ``rng`` before this call)."""
    rng = np.random.default_rng(seed) if rng is None else rng
    seq_lens = np.asarray(seq_lens, dtype=np.int32)
    q_lens = np.asarray(q_lens, dtype=np.int32)
    B = int(seq_lens.shape[0])
    assert q_lens.shape == (B,) and np.all(q_lens <= seq_lens) and np.all(q_lens >= 0)
    if is_decode is None:
        is_decode = q_lens == 1
    is_decode = np.asarray(is_decode, dtype=bool)
    Hkv, Hq, D, bs = num_kv_heads, num_q_heads, head_size, block_size

    # 2. block permutation
    pages = (seq_lens.astype(np.int64) + bs - 1) // bs
    need = int(pages.sum())
    if num_blocks is None:
        num_blocks = max(1, int(math.ceil(need * 1.1)))
    assert num_blocks >= need
    perm = rng.permutation(num_blocks).astype(np.int32)
    max_pages = int(max(1, pages.max(initial=1)))
    block_table = np.full((B, max_pages), -1, dtype=np.int32)
    pos = 0
    for b in range(B):
        n = int(pages[b])
        block_table[b, :n] = perm[pos: pos + n]
        pos += n

    # 3. outliers / magnitudes
    k_out = np.ones(Hkv * D, np.float32)
    v_out = np.ones(Hkv * D, np.float32)
    if k_outlier_frac > 0:
        n = int(round(k_outlier_frac * Hkv * D))
        k_out[rng.choice(Hkv * D, size=n, replace=False)] = k_outlier_gain
    if v_outlier_frac > 0:
        n = int(round(v_outlier_frac * Hkv * D))
        v_out[rng.choice(Hkv * D, size=n, replace=False)] = v_outlier_gain
    k_out = k_out.reshape(Hkv, D)
    v_out = v_out.reshape(Hkv, D)
    total = int(seq_lens.astype(np.int64).sum())
    if token_lognormal_sigma > 0:
        k_mag = rng.lognormal(0.0, token_lognormal_sigma, size=total).astype(np.float32)
        v_mag = rng.lognormal(0.0, token_lognormal_sigma, size=total).astype(np.float32)
    else:
        k_mag = v_mag = None

    off = np.zeros(B + 1, np.int64)
    off[1:] = np.cumsum(seq_lens.astype(np.int64))

    # 4. K, V, Q — one sequence at a time
    def draw_kv(out_gain, mag):
        out = np.empty((total, Hkv, D), np.uint16)
        for b in range(B):
            lo, hi = int(off[b]), int(off[b + 1])
            x = rng.standard_normal((hi - lo, Hkv, D), dtype=np.float32)
            x *= out_gain[None]
            if mag is not None:
                x *= mag[lo:hi, None, None]
            out[lo:hi] = _to_bf16_bits(x)
        return out

    key = draw_kv(k_out, k_mag)
    value = draw_kv(v_out, v_mag)
    cu_q = np.zeros(B + 1, np.int32)
    cu_q[1:] = np.cumsum(q_lens)
    query = np.empty((int(cu_q[-1]), Hq, D), np.uint16)
    for b in range(B):
        lo, hi = int(cu_q[b]), int(cu_q[b + 1])
        query[lo:hi] = _to_bf16_bits(rng.standard_normal((hi - lo, Hq, D), dtype=np.float32))

    slot = np.empty(total, np.int64)
    for b in range(B):
        t = np.arange(int(seq_lens[b]), dtype=np.int64)
        slot[off[b]: off[b + 1]] = block_table[b, t // bs].astype(np.int64) * bs + t % bs

    two688 = np.float32(6.0 * 448.0)
    k_scale = np.float32(_bf16_bits_absmax(key) / two688)
    v_scale = np.float32(_bf16_bits_absmax(value) / two688)
    if k_scale == 0:
        k_scale = np.float32(1.0)
    if v_scale == 0:
        v_scale = np.float32(1.0)
    return Workload(name=name, seed=seed, num_q_heads=Hq, num_kv_heads=Hkv, head_size=D,
                    block_size=bs, num_blocks=num_blocks, seq_lens=seq_lens, q_lens=q_lens,
                    is_decode=is_decode, block_table=block_table, token_offsets=off,
                    key=key, value=value, query=query, cu_q=cu_q, slot_mapping=slot,
                    k_scale=k_scale, v_scale=v_scale)


def make_config(cfg: int, scale: float = 1.0) -> Workload:
    """The five benchmark configurations (seed = config number).

    ``scale`` < 1 shrinks lengths and batch for quick CPU work while keeping
    head geometry, block size and value distributions.
    """
    rng = np.random.default_rng(cfg)
    name = CONFIG_NAMES[cfg]
    if cfg == 1:
        lens = np.array([37, 64], np.int32)
        return make_workload(seed=cfg, name=name, rng=rng, seq_lens=lens, q_lens=np.ones(2, np.int32),
                             num_q_heads=4, num_kv_heads=2, head_size=64, block_size=16,
                             num_blocks=12)
    if cfg == 2:
        B = max(1, int(round(32 * scale)))
        lens = rng.integers(512, 2049, size=B).astype(np.int32)
        if scale < 1:
            lens = np.maximum(2, (lens * scale).astype(np.int32))
        return make_workload(seed=cfg, name=name, rng=rng, seq_lens=lens, q_lens=np.ones(B, np.int32),
                             num_q_heads=16, num_kv_heads=8, head_size=128, block_size=16,
                             k_outlier_frac=0.02, k_outlier_gain=8.0,
                             v_outlier_frac=0.02, v_outlier_gain=8.0)
    if cfg == 3:
        B = max(1, int(round(8 * scale)))
        L = max(2, int(32768 * scale))
        lens = np.full(B, L, np.int32)
        return make_workload(seed=cfg, name=name, rng=rng, seq_lens=lens, q_lens=np.ones(B, np.int32),
                             num_q_heads=32, num_kv_heads=8, head_size=128, block_size=16,
                             token_lognormal_sigma=0.5)
    if cfg == 4:
        B = max(1, int(round(4 * scale)))
        new = max(1, int(2048 * scale))
        cached = int(8192 * scale)
        lens = np.full(B, cached + new, np.int32)
        return make_workload(seed=cfg, name=name, rng=rng, seq_lens=lens,
                             q_lens=np.full(B, new, np.int32), is_decode=np.zeros(B, bool),
                             num_q_heads=32, num_kv_heads=8, head_size=128, block_size=32)
    if cfg == 5:
        B = max(2, int(round(256 * scale)))
        lens = np.clip(np.round(np.exp(rng.normal(math.log(1500.0), 1.0, size=B))), 16, 65536)
        if scale < 1:
            lens = np.maximum(16, np.round(lens * scale))
        lens = lens.astype(np.int32)
        order = rng.permutation(B)
        is_decode = np.zeros(B, bool)
        is_decode[order[: B // 2]] = True
        q_lens = np.where(is_decode, 1, np.minimum(128, lens)).astype(np.int32)
        return make_workload(seed=cfg, name=name, rng=rng, seq_lens=lens, q_lens=q_lens,
                             is_decode=is_decode, num_q_heads=16, num_kv_heads=2, head_size=256,
                             block_size=16, k_outlier_frac=0.01, k_outlier_gain=20.0)
    raise ValueError(f"unknown config {cfg}")


def make_activations(seed: int, m: int, k: int, outlier_frac: float = 0.01, outlier_gain: float = 20.0,
                     token_lognormal_sigma: float = 0.5):
    """bf16 activation matrix [m, k] as uint16 bits, and its per-tensor scale
    ``amax / (6 * 448)``. Draw order: outlier channels, per-row magnitudes
    (lognormal), then fp32 standard normal values rounded to bf16."""
    rng = np.random.default_rng(seed)
    gain = np.ones(k, np.float32)
    n_out = int(round(outlier_frac * k))
    if n_out:
        gain[rng.choice(k, n_out, replace=False)] = outlier_gain
    mag = np.exp(rng.normal(0.0, token_lognormal_sigma, size=(m, 1))).astype(np.float32)
    x = rng.standard_normal((m, k), dtype=np.float32) * mag * gain
    bits = _to_bf16_bits(x)
    g = np.float32(_bf16_bits_absmax(bits) / np.float32(6 * 448))
    return bits, (g if g != 0 else np.float32(1.0))


def fp8_kv_scales(w: Workload, kv_dtype: str):
    """Per-tensor kv scales for an FP8 cache of workload w: amax / 448
    (E4M3) or amax / 57344 (E5M2) in fp32 over each whole bf16 tensor, so that
    the largest magnitude lands on the format's largest finite value."""
    top = {"fp8_e4m3": np.float32(448.0), "fp8_e5m2": np.float32(57344.0)}[kv_dtype]
    ks = np.float32(_bf16_bits_absmax(w.key) / top)
    vs = np.float32(_bf16_bits_absmax(w.value) / top)
    return (ks if ks != 0 else np.float32(1.0)), (vs if vs != 0 else np.float32(1.0))
