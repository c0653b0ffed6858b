"""Parity of FP8 (E4M3FN, E5M2) KV caches [P40177 "Key source snippets":
fp8_e4m3 / fp8_e5m2 beside nvfp4] through the same append, dequantize (paged
and page-form), decode and chunked-prefill kernels as NVFP4: stored bytes and
dequantised values bit-exact against the oracle, attention within
|gpu - ref| <= 2e-3 + 1e-2 |ref| of the oracle's fp64 attention on the same
FP8 cache, on the per-pair and split-K decode paths and in prefill."""
import dataclasses

import numpy as np
import pytest
import torch

import bit_quantized_paged_amd as nvk
from oracle import nvfp4_oracle as O
from workloads import fp8_kv_scales, make_config, make_workload
from gpu_util import Dev, assert_attn_close, bf16_to_np, oracle_pool

pytestmark = pytest.mark.gpu

KV = ["fp8_e4m3", "fp8_e5m2"]

CASES = {
    "c1_d64_bs16": lambda: make_config(1),
    "c2_d128_bs16": lambda: make_config(2, scale=0.08),
    "c5_d256_bs16": lambda: make_config(5, scale=0.05),
    "d128_bs64_gqa4": lambda: make_workload(seed=21, name="x", seq_lens=[1, 63, 64, 65, 200, 129],
                                            q_lens=[1, 1, 1, 1, 1, 1], num_q_heads=16, num_kv_heads=4,
                                            head_size=128, block_size=64),
    "d64_bs32_mha": lambda: make_workload(seed=22, name="x", seq_lens=[33, 95, 7], q_lens=[1, 1, 1],
                                          num_q_heads=3, num_kv_heads=3, head_size=64, block_size=32),
}


def _fp8(w, kv):
    ks, vs = fp8_kv_scales(w, kv)
    return dataclasses.replace(w, k_scale=ks, v_scale=vs)


def _decode_rows(w):
    """One decode query per sequence: the last query row of each."""
    if np.all(w.q_lens == 1):
        return w
    qrows = w.cu_q[1:] - 1
    return dataclasses.replace(w, q_lens=np.ones(w.num_seqs, np.int32), query=w.query[qrows],
                               cu_q=np.arange(w.num_seqs + 1, dtype=np.int32))


@pytest.mark.parametrize("layout", ["HND", "NHD"])
@pytest.mark.parametrize("kv", KV)
@pytest.mark.parametrize("name", sorted(CASES))
def test_fp8_append_and_dequant_bitexact(name, kv, layout):
    w = _fp8(CASES[name](), kv)
    d = Dev(w, layout, kv_dtype=kv)
    d.append_all()
    torch.cuda.synchronize()
    ref = oracle_pool(w, kv)
    got = d.pool_logical()
    bad = np.argwhere(got != ref)
    assert bad.size == 0, f"{name}/{kv}/{layout}: {len(bad)} bytes differ, first at {bad[:3].tolist()}"
    ok, ov = d.dequant()
    torch.cuda.synchronize()
    rk, rv = O.dequant_paged(ref, w.block_table, w.seq_lens, w.k_scale, w.v_scale, w.head_size, kv)
    assert np.array_equal(bf16_to_np(ok), rk) and np.array_equal(bf16_to_np(ov), rv)


@pytest.mark.parametrize("kv", KV)
def test_fp8_append_saturates_like_the_oracle(kv):
    """A scale far below amax / max_finite: most values saturate to the
    largest finite code (sign kept), small ones round into subnormals."""
    w = CASES["c2_d128_bs16"]()
    w = dataclasses.replace(w, k_scale=np.float32(w.k_scale) * np.float32(1e-3), v_scale=np.float32(1e-7))
    d = Dev(w, "HND", kv_dtype=kv)
    d.append_all()
    torch.cuda.synchronize()
    assert np.array_equal(d.pool_logical(), oracle_pool(w, kv))


@pytest.mark.parametrize("layout", ["HND", "NHD"])
@pytest.mark.parametrize("kv", KV)
@pytest.mark.parametrize("name", sorted(CASES))
def test_fp8_decode_parity(name, kv, layout):
    w = _decode_rows(_fp8(CASES[name](), kv))
    d = Dev(w, layout, kv_dtype=kv)
    d.append_all()
    out = d.decode()
    torch.cuda.synchronize()
    ref = O.paged_attention(oracle_pool(w, kv), w.query, w.cu_q, w.block_table, w.seq_lens, w.k_scale,
                            w.v_scale, np.float32(d.sm_scale), w.head_size, kv_dtype=kv)
    assert_attn_close(out, ref, f"{name}/{kv}/{layout} decode")


# (head size, q heads, kv heads, block size, batch, longest) with at least one
# (sequence, kv head) pair per CU and lengths the per-pair path takes for FP8
# (8 steps of 32 keys per wave: 12 waves at D = 64, 8 at 128, 4 at 256)
PAIR_CASES = {
    "d128_gqa2_bs16": (128, 16, 8, 16, 32, 2048),
    "d64_gqa4_bs32": (64, 16, 4, 32, 64, 3072),
    "d256_gqa8_bs16": (256, 16, 2, 16, 128, 1024),
}


@pytest.mark.parametrize("kv", KV)
@pytest.mark.parametrize("name", sorted(PAIR_CASES))
def test_fp8_decode_per_pair_and_split(name, kv):
    D, hq, hkv, bs, B, lmax = PAIR_CASES[name]
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert B * hkv >= cus
    rng = np.random.default_rng(43)
    lens = rng.integers(1, lmax + 1, size=B).astype(np.int32)
    lens[:7] = [1, 31, 32, 33, bs - 1, bs + 1, lmax]
    w = make_workload(seed=52, name="pairs", seq_lens=lens, q_lens=np.ones(B, np.int32), num_q_heads=hq,
                      num_kv_heads=hkv, head_size=D, block_size=bs)
    w = dataclasses.replace(w, query=w.query[w.cu_q[1:] - 1], cu_q=np.arange(B + 1, dtype=np.int32))
    w = _fp8(w, kv)
    mb = w.block_table.shape[1]
    assert nvk.decode_plan(B, hkv, D, bs, mb, int(lens.max()), kv) == nvk.DECODE_PER_PAIR
    d = Dev(w, "HND", kv_dtype=kv)
    d.append_all()
    out = d.decode()
    torch.cuda.synchronize()
    ref = O.paged_attention(oracle_pool(w, kv), w.query, w.cu_q, w.block_table, w.seq_lens, w.k_scale, w.v_scale,
                            np.float32(d.sm_scale), D, kv_dtype=kv)
    assert_attn_close(out, ref, f"{name}/{kv} per pair")
    wide = np.pad(w.block_table, ((0, 0), (0, (lmax * 4) // bs)), constant_values=0)
    assert nvk.decode_plan(B, hkv, D, bs, wide.shape[1], 0, kv) == nvk.DECODE_SPLIT_K
    d.bt = torch.from_numpy(np.ascontiguousarray(wide, dtype=np.int32)).cuda()
    out_split = d.decode(max_seq_len=0)
    torch.cuda.synchronize()
    assert_attn_close(out_split, ref, f"{name}/{kv} split-K")


@pytest.mark.parametrize("kv", KV)
def test_fp8_decode_long_sequences(kv):
    w = _fp8(make_workload(seed=33, name="long", seq_lens=[16384, 9001, 1], q_lens=[1, 1, 1], num_q_heads=32,
                           num_kv_heads=8, head_size=128, block_size=16), kv)
    d = Dev(w, "HND", kv_dtype=kv)
    d.append_all()
    out = d.decode()
    torch.cuda.synchronize()
    ref = O.paged_attention(oracle_pool(w, kv), w.query, w.cu_q, w.block_table, w.seq_lens, w.k_scale, w.v_scale,
                            np.float32(d.sm_scale), 128, kv_dtype=kv)
    assert_attn_close(out, ref, f"{kv} long")


@pytest.mark.parametrize("kv", KV)
def test_fp8_decode_fp8_output_and_graph_replays(kv):
    """FP8 cache in, FP8-E4M3 output out (within half an E4M3 step plus the
    attention tolerance); the bf16 decode captured in a HIP graph reproduces
    the eager result on every replay, with eager work between replays."""
    from test_gpu_parity import _fp8_close
    w = _fp8(make_workload(seed=34, name="g", seq_lens=[700, 33, 4000, 129], q_lens=[1, 1, 1, 1],
                           num_q_heads=16, num_kv_heads=8, head_size=128, block_size=16), kv)
    d = Dev(w, "HND", kv_dtype=kv)
    d.append_all()
    ref = O.paged_attention(oracle_pool(w, kv), w.query, w.cu_q, w.block_table, w.seq_lens, w.k_scale, w.v_scale,
                            np.float32(d.sm_scale), 128, kv_dtype=kv)
    ws = torch.zeros(nvk.decode_workspace_size(w.num_seqs, 16, 8, 128), dtype=torch.uint8, device="cuda")
    codes = torch.empty((w.num_seqs, 16, 128), dtype=torch.uint8, device="cuda")
    os_t = torch.tensor([0.0625], dtype=torch.float32, device="cuda")
    nvk.paged_attention_decode(d.pool, d.query, d.bt, d.seq_lens, int(w.seq_lens.max()), d.k_scale, d.v_scale,
                               d.sm_scale, codes, ws, o_scale=os_t)
    torch.cuda.synchronize()
    _fp8_close(codes, ref, 0.0625, f"{kv} decode fp8 out")

    eager = d.decode(ws=ws)
    torch.cuda.synchronize()
    assert_attn_close(eager, ref, f"{kv} eager")
    out = torch.zeros_like(eager)
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(st):
        with torch.cuda.graph(g, stream=st):
            nvk.paged_attention_decode(d.pool, d.query, d.bt, d.seq_lens, int(w.seq_lens.max()), d.k_scale,
                                       d.v_scale, d.sm_scale, out, ws)
    torch.cuda.current_stream().wait_stream(st)
    for k in range(3):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {k}"
        again = d.decode(ws=ws)
        torch.cuda.synchronize()
        assert torch.equal(again, eager)


PREFILL_CASES = {
    "c4_d128_bs32": lambda: make_config(4, scale=0.06),
    "c5_d256_bs16": lambda: make_config(5, scale=0.05),
    "d128_bs64_gqa4": lambda: make_workload(seed=21, name="x", seq_lens=[1, 63, 64, 65, 200, 129],
                                            q_lens=[1, 1, 5, 1, 17, 3], num_q_heads=16, num_kv_heads=4,
                                            head_size=128, block_size=64),
    "d64_bs32_mha": lambda: make_workload(seed=22, name="x", seq_lens=[33, 95, 7], q_lens=[1, 40, 7],
                                          num_q_heads=3, num_kv_heads=3, head_size=64, block_size=32),
}


@pytest.mark.parametrize("split", [False, True], ids=["grid", "split"])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("kv", KV)
@pytest.mark.parametrize("name", sorted(PREFILL_CASES))
def test_fp8_prefill_parity(name, kv, causal, split):
    w = _fp8(PREFILL_CASES[name](), kv)
    d = Dev(w, "NHD" if causal else "HND", kv_dtype=kv)
    d.append_all()
    out = d.prefill(causal=causal, split=split)
    torch.cuda.synchronize()
    ref = O.paged_attention(oracle_pool(w, kv), w.query, w.cu_q, w.block_table, w.seq_lens, w.k_scale, w.v_scale,
                            np.float32(d.sm_scale), w.head_size, causal=causal, kv_dtype=kv)
    assert_attn_close(out, ref, f"{name}/{kv}/causal={causal} split={split} prefill")


@pytest.mark.parametrize("kv", KV)
def test_fp8_prefill_split_long(kv):
    """An FP8 cache through the key split with jobs long enough to be cut
    (the part records hold the same state as for NVFP4)."""
    w = _fp8(make_workload(seed=31, name="x", seq_lens=[3000, 900, 40], q_lens=[64, 30, 40], num_q_heads=8,
                           num_kv_heads=2, head_size=128, block_size=16), kv)
    d = Dev(w, "HND", kv_dtype=kv)
    d.append_all()
    out = d.prefill(split=True)
    torch.cuda.synchronize()
    parts = d.prefill_ws()[:w.num_seqs * 32].view(torch.int32).view(-1, 8)[:, 1]
    assert int(parts.max()) > 1, "no rank was cut"
    ref = O.paged_attention(oracle_pool(w, kv), w.query, w.cu_q, w.block_table, w.seq_lens, w.k_scale, w.v_scale,
                            np.float32(d.sm_scale), w.head_size, kv_dtype=kv)
    assert_attn_close(out, ref, f"{kv} split prefill")


@pytest.mark.parametrize("kv", KV)
def test_fp8_prefill_with_fp8_output(kv):
    """FP8 cache in, FP8-E4M3 attention output out: decoded codes within half
    an E4M3 step of the reference plus the attention tolerance."""
    from test_gpu_parity import _fp8_close
    w = _fp8(PREFILL_CASES["c4_d128_bs32"](), kv)
    d = Dev(w, "HND", kv_dtype=kv)
    d.append_all()
    os = 0.03125
    codes = d.prefill(o_scale=os)
    torch.cuda.synchronize()
    ref = O.paged_attention(oracle_pool(w, kv), w.query, w.cu_q, w.block_table, w.seq_lens, w.k_scale, w.v_scale,
                            np.float32(d.sm_scale), w.head_size, kv_dtype=kv)
    _fp8_close(codes, ref, os, f"{kv} prefill fp8 out")


@pytest.mark.parametrize("kv", KV)
@pytest.mark.parametrize("name", ["c2_d128_bs16", "c5_d256_bs16", "d64_bs32_mha"])
def test_fp8_dequant_pages_bitexact(name, kv):
    """Page-form dequantize of an FP8 cache: all pages, then a subset with
    repeats and ids outside the pool (skipped); unlisted pages untouched."""
    from test_gpu_parity import _bf16_sentinel
    w = _fp8(CASES[name](), kv)
    nb, bs, hkv, D = w.num_blocks, w.block_size, w.num_kv_heads, w.head_size
    d = Dev(w, "NHD", kv_dtype=kv)
    d.append_all()
    out = _bf16_sentinel((nb, 2, hkv, bs, D)).permute(0, 1, 3, 2, 4)
    nvk.dequant_pages(d.pool, None, d.k_scale, d.v_scale, out)
    torch.cuda.synchronize()
    ref = O.dequant_pages(oracle_pool(w, kv), np.arange(nb), w.k_scale, w.v_scale, D, kv)
    assert np.array_equal(bf16_to_np(out), ref), name
    ids = np.array([nb - 1, 0, -1, nb, min(2, nb - 1)], np.int32)
    out2 = _bf16_sentinel((nb, 2, bs, hkv, D))
    nvk.dequant_pages(d.pool, torch.from_numpy(ids).cuda(), d.k_scale, d.v_scale, out2)
    torch.cuda.synchronize()
    got = bf16_to_np(out2)
    listed = sorted({int(p) for p in ids if 0 <= p < nb})
    assert np.array_equal(got[listed], ref[listed])
    rest = [p for p in range(nb) if p not in listed]
    assert np.all(got[rest] == 0xFFFF)
