"""Pins of the oracle's paged attention and paged dequantize: torch's fp64
scaled-dot-product attention on the dequantised cache, pure-Python loops on
tiny inputs, and invariants (block placement, constant values, one key,
causal prefix)."""
import math

import numpy as np
import pytest
import torch

from oracle import nvfp4_oracle as O
from workloads import make_workload


def _build(seed, lens, q_lens, hq, hkv, D, bs, num_blocks=None, **kw):
    w = make_workload(seed=seed, name="t", seq_lens=lens, q_lens=q_lens, num_q_heads=hq,
                      num_kv_heads=hkv, head_size=D, block_size=bs, num_blocks=num_blocks, **kw)
    pool = np.zeros(O.pool_shape(w.num_blocks, bs, hkv, D), np.uint8)
    O.append(pool, w.key, w.value, w.slot_mapping, w.k_scale, w.v_scale)
    return w, pool


def _dense_kv(w, pool, b):
    L = int(w.seq_lens[b])
    K = O.dequantize_rows(O.gather_rows(pool, w.block_table[b], L, 0), w.k_scale, w.head_size)
    V = O.dequantize_rows(O.gather_rows(pool, w.block_table[b], L, 1), w.v_scale, w.head_size)
    return K.astype(np.float64), V.astype(np.float64)


@pytest.mark.parametrize("causal", [True, False])
def test_attention_matches_torch_sdpa(causal):
    lens, qls = [37, 64, 5, 33], [1, 3, 5, 17]
    w, pool = _build(11, lens, qls, 8, 2, 64, 16)
    sm = np.float32(1.0 / 8.0)
    out = O.paged_attention(pool, w.query, w.cu_q, w.block_table, w.seq_lens, w.k_scale, w.v_scale,
                            sm, 64, causal=causal)
    G = 4
    for b in range(len(lens)):
        K, V = _dense_kv(w, pool, b)
        L, nq = lens[b], qls[b]
        q = torch.from_numpy(O.bf16_to_f32(w.query[w.cu_q[b]: w.cu_q[b + 1]]).astype(np.float64))
        q = q.permute(1, 0, 2)                                          # [Hq, nq, D]
        k = torch.from_numpy(K).permute(1, 0, 2).repeat_interleave(G, 0)  # [Hq, L, D]
        v = torch.from_numpy(V).permute(1, 0, 2).repeat_interleave(G, 0)
        if causal:
            i = torch.arange(nq)[:, None]
            j = torch.arange(L)[None, :]
            mask = j <= (L - nq + i)      # bottom-right aligned
        else:
            mask = torch.ones(nq, L, dtype=torch.bool)
        ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=mask, scale=float(sm))
        got = out[w.cu_q[b]: w.cu_q[b + 1]].transpose(1, 0, 2)
        np.testing.assert_allclose(got, ref.numpy(), rtol=1e-12, atol=1e-12)


def test_attention_bruteforce_loops():
    lens, qls = [5, 3], [2, 1]
    w, pool = _build(12, lens, qls, 4, 2, 64, 16, num_blocks=3)
    sm = np.float32(0.125)
    out = O.paged_attention(pool, w.query, w.cu_q, w.block_table, w.seq_lens, w.k_scale, w.v_scale, sm, 64)
    for b in range(2):
        K, V = _dense_kv(w, pool, b)
        L, nq = lens[b], qls[b]
        for i in range(nq):
            qrow = w.cu_q[b] + i
            for h in range(4):
                kvh = h // 2
                q = [float(t) for t in O.bf16_to_f32(w.query[qrow, h])]
                lim = L - nq + i
                scores = []
                for j in range(lim + 1):
                    scores.append(sum(q[d] * float(K[j, kvh, d]) for d in range(64)) * float(sm))
                mx = max(scores)
                ws = [math.exp(s - mx) for s in scores]
                tot = sum(ws)
                for d in range(64):
                    want = sum(ws[j] * float(V[j, kvh, d]) for j in range(lim + 1)) / tot
                    assert abs(out[qrow, h, d] - want) <= 1e-12 * max(1.0, abs(want))


def test_attention_invariant_to_block_placement():
    lens, qls = [40, 19], [1, 4]
    w, pool = _build(13, lens, qls, 4, 2, 128, 16, num_blocks=8)
    sm = np.float32(0.088)
    a = O.paged_attention(pool, w.query, w.cu_q, w.block_table, w.seq_lens, w.k_scale, w.v_scale, sm, 128)
    # move every used block to a new physical index
    perm = np.random.default_rng(0).permutation(w.num_blocks)
    pool2 = np.zeros_like(pool)
    pool2[perm] = pool
    bt2 = np.where(w.block_table >= 0, perm[np.maximum(w.block_table, 0)], -1).astype(np.int32)
    b = O.paged_attention(pool2, w.query, w.cu_q, bt2, w.seq_lens, w.k_scale, w.v_scale, sm, 128)
    assert np.array_equal(a, b)


def test_constant_values_and_single_key():
    lens, qls = [23, 1], [1, 1]
    w, pool = _build(14, lens, qls, 2, 1, 64, 16, num_blocks=3)
    # overwrite every V row with one constant quantised row
    row = O.quantize_rows(w.value[:1, 0], w.v_scale)[0]
    pool[:, 1] = row
    out = O.paged_attention(pool, w.query, w.cu_q, w.block_table, w.seq_lens, w.k_scale, w.v_scale,
                            np.float32(0.3), 64)
    vhat = O.dequantize_rows(row[None], w.v_scale, 64)[0].astype(np.float64)
    np.testing.assert_allclose(out[0], np.broadcast_to(vhat, (2, 64)), rtol=1e-13, atol=1e-15)
    # sequence 1 has a single key: the output is exactly that key's value row
    np.testing.assert_array_equal(out[1], np.broadcast_to(vhat, (2, 64)))


def test_causal_prefix_ignores_later_keys():
    lens, qls = [50], [10]
    w, pool = _build(15, lens, qls, 2, 1, 64, 16)
    sm = np.float32(0.125)
    a = O.paged_attention(pool, w.query, w.cu_q, w.block_table, w.seq_lens, w.k_scale, w.v_scale, sm, 64)
    # scramble the last key (position 49): only the last query may change
    j = 49
    blk, row = w.block_table[0, j // 16], j % 16
    pool[blk, :, row] ^= np.uint8(0x5A)
    pool[blk, :, row, :, 32:] = np.uint8(0x30)   # keep scale bytes finite
    b = O.paged_attention(pool, w.query, w.cu_q, w.block_table, w.seq_lens, w.k_scale, w.v_scale, sm, 64)
    assert np.array_equal(a[:9], b[:9])
    assert not np.array_equal(a[9], b[9])


def test_dequant_paged_layout():
    lens = [37, 64, 1]
    w, pool = _build(16, lens, [1, 1, 1], 4, 2, 64, 16, num_blocks=12)
    kd, vd = O.dequant_paged(pool, w.block_table, w.seq_lens, w.k_scale, w.v_scale, 64)
    assert kd.shape == (102, 2, 64) and kd.dtype == np.uint16
    off = 0
    for b, L in enumerate(lens):
        for j in range(L):
            blk, row = w.block_table[b, j // 16], j % 16
            want = O.f32_to_bf16(O.dequantize_rows(pool[blk, 0, row], w.k_scale, 64))
            assert np.array_equal(kd[off + j], want)
            want = O.f32_to_bf16(O.dequantize_rows(pool[blk, 1, row], w.v_scale, 64))
            assert np.array_equal(vd[off + j], want)
        off += L


def test_quantised_attention_close_to_bf16_attention():
    """Band check: attention on the quantised cache stays within a
    quantisation-level distance of attention on the bf16 cache."""
    lens, qls = [300, 129], [1, 1]
    w, pool = _build(17, lens, qls, 8, 2, 128, 16)
    sm = np.float32(1 / math.sqrt(128))
    out = O.paged_attention(pool, w.query, w.cu_q, w.block_table, w.seq_lens, w.k_scale, w.v_scale, sm, 128)
    for b in range(2):
        lo, hi = w.token_offsets[b], w.token_offsets[b + 1]
        K = torch.from_numpy(O.bf16_to_f32(w.key[lo:hi]).astype(np.float64)).permute(1, 0, 2).repeat_interleave(4, 0)
        V = torch.from_numpy(O.bf16_to_f32(w.value[lo:hi]).astype(np.float64)).permute(1, 0, 2).repeat_interleave(4, 0)
        q = torch.from_numpy(O.bf16_to_f32(w.query[b:b + 1]).astype(np.float64)).permute(1, 0, 2)
        ref = torch.nn.functional.scaled_dot_product_attention(q, K, V, scale=float(sm)).permute(1, 0, 2).numpy()
        err = np.abs(out[b:b + 1] - ref).max()
        # E2M1 relative half-step is up to 1/6 of the block amax; averaged over
        # hundreds of keys the output error is far smaller than the value scale
        assert err < 0.25, err
        assert err > 1e-4, "quantisation must be visible"
