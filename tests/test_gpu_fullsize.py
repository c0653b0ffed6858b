"""Parity at the full sizes of the four benchmark workloads (small-model
decode, long-context decode, chunked prefill, mixed serving batch), in the
launch configuration the benchmark times: an HND pool filled with the cached
prefix, then one append of the new tokens, decode over the 1-token sequences
and chunked prefill over the rest, with the same batch splits and length
hints. The oracle quantises every token of the workload itself and then
checks:

- the whole pool, bit-exact;
- the whole decode output (every head of every decode sequence);
- prefill: the whole output of the mixed batch's prefill half; for the
  2048-token chunks, 64-row runs of every sequence at the chunk's start, at
  its end and across a workgroup tile boundary in its middle (each run is
  the last 64 queries of a sequence cut after the run's last token, which
  is what bottom-right causal alignment makes it);
- the paged dequantize of the decode batch and the page-form dequantize of
  its pages, as the benchmark runs them, on sampled sequences, bit-exact.
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
        wsp = torch.zeros(nvk.prefill_workspace_size(D), dtype=torch.uint8, device=dev)  # key split, as timed
        nvk.paged_attention_prefill(pool, bf16_dev(wp.query, dev), i32_dev(wp.cu_q, dev), int(wp.q_lens.max()),
                                    i32_dev(wp.block_table, dev), i32_dev(wp.seq_lens, dev), int(wp.seq_lens.max()),
                                    ks, vs, sm, outp, workspace=wsp)
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
    """The longest, the shortest and n_random other sequences of idx (with
    equal lengths: n_random + 1 distinct sequences)."""
    if len(idx) == 0:
        return []
    pick = {int(idx[np.argmax(lens[idx])]), int(idx[np.argmin(lens[idx])])}
    rest = [int(b) for b in idx if int(b) not in pick]
    if rest:
        pick.update(int(b) for b in rng.choice(rest, size=min(n_random, len(rest)), replace=False))
    return sorted(pick)


def prefill_runs(L, nq, run=64, tile_tokens=32):
    """Query-row runs [a, a + n) of a chunk of nq queries: its start, its end,
    and one across the workgroup tile boundary nearest its middle (a tile is
    tile_tokens chunk tokens); the whole chunk when it is short."""
    if nq <= 3 * run:
        return [(0, nq)]
    mid = (nq // 2) // tile_tokens * tile_tokens
    starts = sorted({0, mid - run // 2, nq - run})
    return [(a, run) for a in starts]


def oracle_rows(ref_pool, w, b, a, n, sm, kv="nvfp4", ks=None, vs=None):
    """The oracle's causal attention for query rows a .. a + n - 1 of
    sequence b's chunk: the last n queries of the sequence cut after key
    L - q_len + a + n - 1."""
    L, nq = int(w.seq_lens[b]), int(w.q_lens[b])
    q0 = int(w.cu_q[b]) + a
    ks = w.k_scale if ks is None else ks
    vs = w.v_scale if vs is None else vs
    return O.paged_attention(ref_pool, w.query[q0:q0 + n], np.array([0, n], np.int32), w.block_table[b:b + 1],
                             np.array([L - nq + a + n], np.int32), ks, vs, sm, w.head_size, kv_dtype=kv)


def pool_bytes(pool):
    """The pool's bytes in logical (num_blocks, 2, block_size, Hkv, row) order."""
    return pool.contiguous().view(torch.uint8).cpu().numpy()


@pytest.mark.parametrize("name", sorted(FULL))
def test_full_size_parity(name):
    cfg = FULL[name]
    w = make_config(cfg)
    dev = torch.device("cuda")
    print(f"full-size parity: {name} ({w.num_seqs} seqs, {int(w.seq_lens.sum())} tokens)", flush=True)
    pool, dec_idx, outd, pre_idx, wp, outp = run_like_bench(w, dev)
    rng = np.random.default_rng(100 + cfg)

    # ---- every packed row: the oracle quantises the whole workload
    ref_pool = np.zeros(O.pool_shape(w.num_blocks, w.block_size, w.num_kv_heads, w.head_size), np.uint8)
    O.append(ref_pool, w.key, w.value, w.slot_mapping, w.k_scale, w.v_scale)
    got_pool = pool_bytes(pool)
    bad = np.argwhere(got_pool != ref_pool)
    assert bad.size == 0, f"{name}: {len(bad)} pool bytes differ, first at {bad[:3].tolist()}"
    del got_pool

    sm = np.float32(1.0 / math.sqrt(w.head_size))
    # ---- decode: the whole output
    if len(dec_idx):
        wd = w.subset(dec_idx)
        ref = O.paged_attention(ref_pool, wd.query, wd.cu_q, wd.block_table, wd.seq_lens, w.k_scale, w.v_scale, sm,
                                w.head_size)
        err = assert_attn_close(outd, ref, f"{name} decode ({wd.num_seqs} sequences)")
        print(f"  decode: {ref.size} outputs, max |err| {err:.2e}", flush=True)

    # ---- paged and page-form dequantize of the decode batch
    sd = sample_seqs(dec_idx, w.seq_lens, rng, 3)
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

    # ---- prefill: short chunks whole, long chunks by runs at both ends and across a tile boundary
    if len(pre_idx):
        if np.all(wp.q_lens <= 192):
            ref = O.paged_attention(ref_pool, wp.query, wp.cu_q, wp.block_table, wp.seq_lens, w.k_scale, w.v_scale,
                                    sm, w.head_size)
            err = assert_attn_close(outp, ref, f"{name} prefill ({wp.num_seqs} sequences)")
            print(f"  prefill: {ref.size} outputs, max |err| {err:.2e}", flush=True)
        else:
            rows = 0
            for k in range(wp.num_seqs):
                L, nq = int(wp.seq_lens[k]), int(wp.q_lens[k])
                for a, n in prefill_runs(L, nq):
                    ref = oracle_rows(ref_pool, wp, k, a, n, sm)
                    r0 = int(wp.cu_q[k]) + a
                    assert_attn_close(outp[r0:r0 + n], ref, f"{name} prefill seq {k} rows {a}..{a + n - 1} of {nq}")
                    rows += n
            print(f"  prefill: {rows} rows of {int(wp.cu_q[-1])}", flush=True)


@pytest.mark.parametrize("name,kv", [("long_decode", "fp8_e4m3"), ("mixed_serving", "fp8_e4m3"),
                                     ("mixed_serving", "fp8_e5m2")])
def test_full_size_fp8_decode(name, kv):
    """FP8 caches at full size through the split decode kernel (D = 128 and
    D = 256): the whole batch appended into an FP8 pool, the decode
    sequences decoded in one call, the whole output against the oracle on
    its own FP8 pool of the same tokens."""
    cfg = FULL[name]
    w = make_config(cfg)
    dev = torch.device("cuda")
    print(f"full-size FP8 decode: {name} {kv}", flush=True)
    ksc, vsc = fp8_kv_scales(w, kv)
    ks, vs = scale_dev(ksc, dev), scale_dev(vsc, dev)
    pool = nvk.alloc_pool(w.num_blocks, w.block_size, w.num_kv_heads, w.head_size, "HND", dev, kv_dtype=kv)
    dec_idx = np.nonzero(w.q_lens == 1)[0]
    wd = w.subset(dec_idx)
    nvk.append(pool, bf16_dev(wd.key, dev), bf16_dev(wd.value, dev), i64_dev(wd.slot_mapping, dev), ks, vs)
    Hq, Hkv, D = w.num_q_heads, w.num_kv_heads, w.head_size
    assert nvk.decode_plan(wd.num_seqs, Hkv, D, w.block_size, wd.block_table.shape[1], int(wd.seq_lens.max()),
                           kv) == nvk.DECODE_SPLIT_K
    out = torch.empty((wd.num_seqs, Hq, D), dtype=torch.bfloat16, device=dev)
    ws = torch.zeros(nvk.decode_workspace_size(wd.num_seqs, Hq, Hkv, D), dtype=torch.uint8, device=dev)
    sm = np.float32(1.0 / math.sqrt(D))
    nvk.paged_attention_decode(pool, bf16_dev(wd.query, dev), i32_dev(wd.block_table, dev), i32_dev(wd.seq_lens, dev),
                               int(wd.seq_lens.max()), ks, vs, float(sm), out, ws)
    torch.cuda.synchronize()
    ref_pool = np.zeros(O.pool_shape(w.num_blocks, w.block_size, Hkv, D, kv), np.uint8)
    O.append(ref_pool, wd.key, wd.value, wd.slot_mapping, ksc, vsc, kv)
    assert np.array_equal(pool_bytes(pool), ref_pool), f"{name} {kv}: pool bytes differ"
    ref = O.paged_attention(ref_pool, wd.query, wd.cu_q, wd.block_table, wd.seq_lens, ksc, vsc, sm, D, kv_dtype=kv)
    assert_attn_close(out, ref, f"{name} {kv} decode ({wd.num_seqs} sequences)")


def test_full_size_fp8_chunked_prefill():
    """An E4M3 cache at the full chunked-prefill size: 8192 cached tokens per
    sequence appended, then the 2048-token chunks, and one causal prefill
    call; 64-row runs of every sequence (chunk start, end, a tile boundary)
    against the oracle."""
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
    ref_pool = np.zeros(O.pool_shape(w.num_blocks, w.block_size, w.num_kv_heads, D, kv), np.uint8)
    O.append(ref_pool, w.key, w.value, w.slot_mapping, ksc, vsc, kv)
    for b in range(w.num_seqs):
        for a, n in prefill_runs(int(w.seq_lens[b]), int(w.q_lens[b])):
            ref = oracle_rows(ref_pool, w, b, a, n, sm, kv, ksc, vsc)
            r0 = int(w.cu_q[b]) + a
            assert_attn_close(out[r0:r0 + n], ref, f"chunked_prefill {kv} seq {b} rows {a}..{a + n - 1}")
