"""Parity at the full sizes of the four benchmark workloads (small-model
decode, long-context decode, chunked prefill, mixed serving batch), in the
launch configuration the benchmark times: an HND pool filled with the cached
prefix, then one append of the new tokens, decode over the 1-token sequences
and chunked prefill over the rest, with the same batch splits and length
hints. The oracle computes a sample of the outputs one by one:

- packed rows: every token of the sampled sequences plus a random sample of
  all tokens, bit-exact against the oracle's own quantisation;
- decode: every head of the sampled sequences (the longest, the shortest and
  random ones);
- prefill: single query rows of the sampled sequences (first, last and random
  positions), each as a one-query sequence over its causal prefix (the key
  limit L - q_len + i of bottom-right alignment);
- the paged dequantize of the decode batch and the page-form dequantize of
  its pages, as the benchmark runs them: the sampled sequences' rows and
  pages, bit-exact.
"""
import math

import numpy as np
import pytest
import torch

import bit_quantized_paged_amd as nvk
from oracle import nvfp4_oracle as O
from workloads import fp8_kv_scales, make_config
from gpu_util import assert_attn_close, bf16_dev, i32_dev, i64_dev, scale_dev

pytestmark = pytest.mark.gpu

FULL = {"small_decode": 2, "long_decode": 3, "chunked_prefill": 4, "mixed_serving": 5}


def run_like_bench(w, dev):
    """The benchmark's step on one pool: fill, append, decode, prefill."""
    Hq, Hkv, D, bs = w.num_q_heads, w.num_kv_heads, w.head_size, w.block_size
    fd = D // 2 + D // 16
    sm = 1.0 / math.sqrt(D)
    ks, vs = scale_dev(w.k_scale, dev), scale_dev(w.v_scale, dev)
    base = torch.zeros((w.num_blocks, 2, Hkv, bs, fd), dtype=torch.uint8, device=dev)
    pool = base.permute(0, 1, 3, 2, 4)  # logical (num_blocks, 2, bs, Hkv, fd), HND in memory
    cached = w.cached_mask()
    for sel in (cached, ~cached):
        if sel.any():
            nvk.append(pool, bf16_dev(w.key[sel], dev), bf16_dev(w.value[sel], dev), i64_dev(w.slot_mapping[sel], dev),
                       ks, vs)
    dec_idx = np.nonzero(w.q_lens == 1)[0]
    pre_idx = np.nonzero(w.q_lens != 1)[0]
    outd = outp = None
    if len(dec_idx):
        wd = w.subset(dec_idx)
        outd = torch.empty((wd.num_seqs, Hq, D), dtype=torch.bfloat16, device=dev)
        wsd = torch.zeros(nvk.decode_workspace_size(wd.num_seqs, Hq, Hkv, D), dtype=torch.uint8, device=dev)
        nvk.paged_attention_decode(pool, bf16_dev(wd.query, dev), i32_dev(wd.block_table, dev),
                                   i32_dev(wd.seq_lens, dev), int(wd.seq_lens.max()), ks, vs, sm, outd, wsd)
    wp = None
    if len(pre_idx):
        wp = w.subset(pre_idx)
        outp = torch.empty((int(wp.cu_q[-1]), Hq, D), dtype=torch.bfloat16, device=dev)
        nvk.paged_attention_prefill(pool, bf16_dev(wp.query, dev), i32_dev(wp.cu_q, dev), int(wp.q_lens.max()),
                                    i32_dev(wp.block_table, dev), i32_dev(wp.seq_lens, dev), int(wp.seq_lens.max()),
                                    ks, vs, sm, outp)
    torch.cuda.synchronize()
    return pool, dec_idx, outd, pre_idx, wp, outp


def dequant_like_bench(w, pool, dec_idx, dev):
    """The benchmark's two dequantize calls over the decode batch: gathered
    rows per sequence, and every page the batch uses."""
    wd = w.subset(dec_idx)
    Hkv, D, bs = w.num_kv_heads, w.head_size, w.block_size
    ks, vs = scale_dev(w.k_scale, dev), scale_dev(w.v_scale, dev)
    cu = np.zeros(wd.num_seqs, np.int32)
    cu[1:] = np.cumsum(wd.seq_lens)[:-1]
    ok = torch.empty((int(wd.seq_lens.sum()), Hkv, D), dtype=torch.bfloat16, device=dev)
    ov = torch.empty_like(ok)
    nvk.dequant_paged(pool, i32_dev(wd.block_table, dev), i32_dev(wd.seq_lens, dev), i32_dev(cu, dev),
                      int(wd.seq_lens.max()), ks, vs, ok, ov)
    used = np.unique(np.concatenate([wd.block_table[b, :(int(wd.seq_lens[b]) + bs - 1) // bs]
                                     for b in range(wd.num_seqs)])).astype(np.int32)
    pages = torch.empty((w.num_blocks, 2, bs, Hkv, D), dtype=torch.bfloat16, device=dev)
    nvk.dequant_pages(pool, i32_dev(used, dev), ks, vs, pages)
    torch.cuda.synchronize()
    return cu, ok, ov, pages


def sample_seqs(idx, lens, rng, n_random):
    """The longest, the shortest and n_random other sequences of idx."""
    if len(idx) == 0:
        return []
    pick = {int(idx[np.argmax(lens[idx])]), int(idx[np.argmin(lens[idx])])}
    rest = [int(b) for b in idx if int(b) not in pick]
    if rest:
        pick.update(int(b) for b in rng.choice(rest, size=min(n_random, len(rest)), replace=False))
    return sorted(pick)


@pytest.mark.parametrize("name", sorted(FULL))
def test_full_size_sampled_parity(name):
    cfg = FULL[name]
    w = make_config(cfg)
    dev = torch.device("cuda")
    print(f"full-size parity: {name} ({w.num_seqs} seqs, {int(w.seq_lens.sum())} tokens)", flush=True)
    pool, dec_idx, outd, pre_idx, wp, outp = run_like_bench(w, dev)
    rng = np.random.default_rng(100 + cfg)
    sd = sample_seqs(dec_idx, w.seq_lens, rng, 2)
    sp = sample_seqs(pre_idx, w.seq_lens, rng, 1)
    assert sd or sp

    # ---- packed rows of the sampled sequences' tokens and of a random token sample
    off = w.token_offsets
    toks = [np.arange(off[b], off[b + 1]) for b in sd + sp]
    toks.append(rng.choice(int(off[-1]), size=4096, replace=False))
    toks = np.unique(np.concatenate(toks))
    ref_pool = np.zeros(O.pool_shape(w.num_blocks, w.block_size, w.num_kv_heads, w.head_size), np.uint8)
    O.append(ref_pool, w.key[toks], w.value[toks], w.slot_mapping[toks], w.k_scale, w.v_scale)
    slots = w.slot_mapping[toks]
    blk, row = slots // w.block_size, slots % w.block_size
    got_rows = pool[torch.from_numpy(blk).to(dev), :, torch.from_numpy(row).to(dev)].cpu().numpy()
    ref_rows = ref_pool[blk, :, row]
    bad = np.nonzero(np.any(got_rows != ref_rows, axis=(1, 2, 3)))[0]
    assert bad.size == 0, f"{name}: {bad.size} of {toks.size} sampled tokens differ (first token {toks[bad[0]]})"

    sm = np.float32(1.0 / math.sqrt(w.head_size))
    # ---- decode: every head of each sampled sequence
    for b in sd:
        k = int(np.nonzero(dec_idx == b)[0][0])
        q0 = int(w.cu_q[b])
        ref = O.paged_attention(ref_pool, w.query[q0:q0 + 1], np.array([0, 1], np.int32), w.block_table[b:b + 1],
                                w.seq_lens[b:b + 1], w.k_scale, w.v_scale, sm, w.head_size)
        assert_attn_close(outd[k:k + 1], ref, f"{name} decode seq {b} (len {int(w.seq_lens[b])})")

    # ---- paged and page-form dequantize of the decode batch
    if sd:
        cu, ok, ov, pages = dequant_like_bench(w, pool, dec_idx, dev)
        bs = w.block_size
        for b in sd:
            k = int(np.nonzero(dec_idx == b)[0][0])
            L = int(w.seq_lens[b])
            kd, vd = O.dequant_paged(ref_pool, w.block_table[b:b + 1], w.seq_lens[b:b + 1], w.k_scale, w.v_scale,
                                     w.head_size)
            for got, want, nm in ((ok, kd, "K"), (ov, vd, "V")):
                g = got[int(cu[k]):int(cu[k]) + L].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
                assert np.array_equal(g, want), f"{name} dequant {nm} of seq {b} differs"
            ids = w.block_table[b, :(L + bs - 1) // bs].astype(np.int64)
            want_pages = O.dequant_pages(ref_pool, ids, w.k_scale, w.v_scale, w.head_size)
            g = pages[torch.from_numpy(ids).to(dev)].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
            assert np.array_equal(g, want_pages), f"{name} page-form dequant of seq {b}'s pages differs"
        del ok, ov, pages

    # ---- prefill: single query rows over their causal prefix
    for b in sp:
        k = int(np.nonzero(pre_idx == b)[0][0])
        L, nq = int(w.seq_lens[b]), int(w.q_lens[b])
        rows = {0, nq - 1} | {int(i) for i in rng.integers(0, nq, size=2)}
        for i in sorted(rows):
            p = L - nq + i  # absolute position of query row i: it sees keys 0..p
            qi = int(w.cu_q[b]) + i
            ref = O.paged_attention(ref_pool, w.query[qi:qi + 1], np.array([0, 1], np.int32), w.block_table[b:b + 1],
                                    np.array([p + 1], np.int32), w.k_scale, w.v_scale, sm, w.head_size)
            r = int(wp.cu_q[k]) + i
            assert_attn_close(outp[r:r + 1], ref, f"{name} prefill seq {b} row {i} of {nq} (keys 0..{p})")


@pytest.mark.parametrize("name,kv", [("long_decode", "fp8_e4m3"), ("mixed_serving", "fp8_e4m3"),
                                     ("mixed_serving", "fp8_e5m2")])
def test_full_size_fp8_decode_sampled(name, kv):
    """FP8 caches at full size through the split decode kernel (D = 128 and
    D = 256): the whole batch appended into an FP8 pool, the decode
    sequences decoded in one call, sampled sequences against the oracle on
    its own FP8 pool of their tokens."""
    cfg = FULL[name]
    w = make_config(cfg)
    dev = torch.device("cuda")
    print(f"full-size FP8 decode: {name} {kv}", flush=True)
    ksc, vsc = fp8_kv_scales(w, kv)
    ks, vs = scale_dev(ksc, dev), scale_dev(vsc, dev)
    pool = nvk.alloc_pool(w.num_blocks, w.block_size, w.num_kv_heads, w.head_size, "HND", dev, kv_dtype=kv)
    nvk.append(pool, bf16_dev(w.key, dev), bf16_dev(w.value, dev), i64_dev(w.slot_mapping, dev), ks, vs)
    dec_idx = np.nonzero(w.q_lens == 1)[0]
    wd = w.subset(dec_idx)
    Hq, Hkv, D = w.num_q_heads, w.num_kv_heads, w.head_size
    assert nvk.decode_plan(wd.num_seqs, Hkv, D, w.block_size, wd.block_table.shape[1], int(wd.seq_lens.max()),
                           kv) == nvk.DECODE_SPLIT_K
    out = torch.empty((wd.num_seqs, Hq, D), dtype=torch.bfloat16, device=dev)
    ws = torch.zeros(nvk.decode_workspace_size(wd.num_seqs, Hq, Hkv, D), dtype=torch.uint8, device=dev)
    sm = np.float32(1.0 / math.sqrt(D))
    nvk.paged_attention_decode(pool, bf16_dev(wd.query, dev), i32_dev(wd.block_table, dev), i32_dev(wd.seq_lens, dev),
                               int(wd.seq_lens.max()), ks, vs, float(sm), out, ws)
    torch.cuda.synchronize()
    rng = np.random.default_rng(200 + cfg)
    sd = sample_seqs(dec_idx, w.seq_lens, rng, 2)
    off = w.token_offsets
    toks = np.concatenate([np.arange(off[b], off[b + 1]) for b in sd])
    ref_pool = np.zeros(O.pool_shape(w.num_blocks, w.block_size, Hkv, D, kv), np.uint8)
    O.append(ref_pool, w.key[toks], w.value[toks], w.slot_mapping[toks], ksc, vsc, kv)
    for b in sd:
        k = int(np.nonzero(dec_idx == b)[0][0])
        q0 = int(w.cu_q[b])
        ref = O.paged_attention(ref_pool, w.query[q0:q0 + 1], np.array([0, 1], np.int32), w.block_table[b:b + 1],
                                w.seq_lens[b:b + 1], ksc, vsc, sm, D, kv_dtype=kv)
        assert_attn_close(out[k:k + 1], ref, f"{name} {kv} decode seq {b} (len {int(w.seq_lens[b])})")


def test_full_size_fp8_chunked_prefill_sampled():
    """An E4M3 cache at the full chunked-prefill size: 8192 cached tokens per
    sequence appended, then the 2048-token chunks, and one causal prefill
    call; single query rows of sampled sequences against the oracle."""
    kv = "fp8_e4m3"
    w = make_config(FULL["chunked_prefill"])
    dev = torch.device("cuda")
    ksc, vsc = fp8_kv_scales(w, kv)
    ks, vs = scale_dev(ksc, dev), scale_dev(vsc, dev)
    pool = nvk.alloc_pool(w.num_blocks, w.block_size, w.num_kv_heads, w.head_size, "HND", dev, kv_dtype=kv)
    cached = w.cached_mask()
    for sel in (cached, ~cached):
        nvk.append(pool, bf16_dev(w.key[sel], dev), bf16_dev(w.value[sel], dev), i64_dev(w.slot_mapping[sel], dev),
                   ks, vs)
    Hq, D = w.num_q_heads, w.head_size
    sm = np.float32(1.0 / math.sqrt(D))
    out = torch.empty((int(w.cu_q[-1]), Hq, D), dtype=torch.bfloat16, device=dev)
    nvk.paged_attention_prefill(pool, bf16_dev(w.query, dev), i32_dev(w.cu_q, dev), int(w.q_lens.max()),
                                i32_dev(w.block_table, dev), i32_dev(w.seq_lens, dev), int(w.seq_lens.max()),
                                ks, vs, float(sm), out)
    torch.cuda.synchronize()
    rng = np.random.default_rng(300)
    sp = sample_seqs(np.arange(w.num_seqs), w.seq_lens, rng, 1)
    off = w.token_offsets
    toks = np.concatenate([np.arange(off[b], off[b + 1]) for b in sp])
    ref_pool = np.zeros(O.pool_shape(w.num_blocks, w.block_size, w.num_kv_heads, D, kv), np.uint8)
    O.append(ref_pool, w.key[toks], w.value[toks], w.slot_mapping[toks], ksc, vsc, kv)
    for b in sp:
        L, nq = int(w.seq_lens[b]), int(w.q_lens[b])
        for i in sorted({0, nq - 1} | {int(x) for x in rng.integers(0, nq, size=2)}):
            p = L - nq + i
            qi = int(w.cu_q[b]) + i
            ref = O.paged_attention(ref_pool, w.query[qi:qi + 1], np.array([0, 1], np.int32), w.block_table[b:b + 1],
                                    np.array([p + 1], np.int32), ksc, vsc, sm, D, kv_dtype=kv)
            assert_attn_close(out[qi:qi + 1], ref, f"chunked_prefill {kv} seq {b} row {i} (keys 0..{p})")
