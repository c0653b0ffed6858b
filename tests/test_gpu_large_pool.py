"""Pools above 4 GiB. Every kernel forms a block's address as the block id
times the block stride in 64-bit arithmetic and reads within one block
through 32-bit buffer offsets, so the pool itself may exceed any 32-bit
range. Here every block a workload uses lies past byte 4.25 GiB of a pool of
about 4.5 GiB: block ids and slots are shifted by one constant, which changes
no value (the oracle reads the same blocks at their unshifted ids). A 32-bit
wrap would land below the shifted blocks, so the tests also check that
nothing is written there. Writer bytes and dequantised values bit-exact,
attention within |gpu - ref| <= 2e-3 + 1e-2 |ref|, on both decode kernels,
both prefill paths (grid and key split) and an FP8 cache."""
import dataclasses

import numpy as np
import pytest
import torch

import bit_quantized_paged_amd as nvk
from oracle import nvfp4_oracle as O
from workloads import fp8_kv_scales, make_workload
from gpu_util import Dev, assert_attn_close, bf16_to_np, i32_dev, i64_dev, oracle_pool

pytestmark = pytest.mark.gpu

FLOOR = (1 << 32) + (1 << 28)  # byte offset at or past which the first used block starts


@pytest.fixture(autouse=True)
def _release_cached_blocks():
    yield
    torch.cuda.empty_cache()


def _shifted(w, kv="nvfp4", layout="HND"):
    """A Dev whose pool holds `shift` unused blocks ahead of the workload's."""
    d = Dev(w, layout, kv_dtype=kv)
    per_block = d.pool[0].numel() * d.pool.element_size()
    shift = -(-FLOOR // per_block)
    d.pool = nvk.alloc_pool(shift + w.num_blocks, w.block_size, w.num_kv_heads, w.head_size, layout, "cuda",
                            kv_dtype=kv)
    bt = w.block_table.astype(np.int64)
    d.bt = i32_dev(np.where(bt >= 0, bt + shift, -1))
    sm = w.slot_mapping
    d.slots = i64_dev(np.where(sm >= 0, sm + shift * w.block_size, sm))
    d.shift = shift
    assert shift * per_block >= FLOOR
    return d


def _check_writes(d, w, kv="nvfp4"):
    """Nothing below the shifted blocks; the shifted blocks hold the oracle's bytes."""
    assert not bool(d.pool[:d.shift].view(torch.uint8).any()), "a write landed below the workload's blocks"
    got = d.pool[d.shift:].contiguous().view(torch.uint8).cpu().numpy()
    ref = oracle_pool(w, kv)
    bad = np.argwhere(got != ref)
    assert bad.size == 0, f"{len(bad)} bytes differ, first at {bad[:3].tolist()}"


def _fp8(w, kv):
    ks, vs = fp8_kv_scales(w, kv)
    return dataclasses.replace(w, k_scale=ks, v_scale=vs)


def _decode_case(kind):
    if kind == "pair":
        # batch x kv heads above the CU count and at most 22 steps: the per-pair kernel
        rng = np.random.default_rng(61)
        lens = rng.integers(1, 701, size=64).astype(np.int32)
        return make_workload(seed=61, name="x", rng=rng, seq_lens=lens, q_lens=np.ones(64, np.int32),
                             num_q_heads=16, num_kv_heads=8, head_size=128, block_size=16)
    if kind == "split_d128":
        return make_workload(seed=62, name="x", seq_lens=[3000, 129, 1], q_lens=[1, 1, 1], num_q_heads=8,
                             num_kv_heads=2, head_size=128, block_size=16)
    return make_workload(seed=63, name="x", seq_lens=[2000, 40], q_lens=[1, 1], num_q_heads=16, num_kv_heads=2,
                         head_size=256, block_size=16)


# jobs of 63-79 steps: the key split cuts them into two or three parts
PREFILL = {
    "d128": lambda: make_workload(seed=64, name="x", seq_lens=[2500, 90, 700, 5], q_lens=[200, 90, 333, 1],
                                  num_q_heads=8, num_kv_heads=2, head_size=128, block_size=16),
    "d256": lambda: make_workload(seed=65, name="x", seq_lens=[2200, 130], q_lens=[129, 64], num_q_heads=16,
                                  num_kv_heads=2, head_size=256, block_size=16),
}


@pytest.mark.parametrize("kind", ["pair", "split_d128", "split_d256"])
def test_large_pool_append_and_decode(kind):
    w = _decode_case(kind)
    print(f"large pool decode {kind}", flush=True)
    d = _shifted(w)
    d.append_all()
    torch.cuda.synchronize()
    _check_writes(d, w)
    plan = nvk.decode_plan(w.num_seqs, w.num_kv_heads, w.head_size, w.block_size, w.max_blocks_per_seq,
                           int(w.seq_lens.max()))
    assert plan == (nvk.DECODE_PER_PAIR if kind == "pair" else nvk.DECODE_SPLIT_K)
    out = d.decode()
    torch.cuda.synchronize()
    ref = O.paged_attention(oracle_pool(w), w.query, w.cu_q, w.block_table, w.seq_lens, w.k_scale, w.v_scale,
                            np.float32(d.sm_scale), w.head_size)
    assert_attn_close(out, ref, f"large pool decode ({kind})")


@pytest.mark.parametrize("split", [False, True], ids=["grid", "split"])
@pytest.mark.parametrize("kind", sorted(PREFILL))
def test_large_pool_prefill(kind, split):
    w = PREFILL[kind]()
    print(f"large pool prefill {kind} split={split}", flush=True)
    d = _shifted(w)
    d.append_all()
    out = d.prefill(causal=True, split=split)
    torch.cuda.synchronize()
    _check_writes(d, w)
    ref = O.paged_attention(oracle_pool(w), w.query, w.cu_q, w.block_table, w.seq_lens, w.k_scale, w.v_scale,
                            np.float32(d.sm_scale), w.head_size, causal=True)
    assert_attn_close(out, ref, f"large pool prefill ({kind}, split={split})")


def test_large_pool_dequant_both_forms():
    """Sequence form through the shifted block table; page form by the shifted
    page ids into a bf16 page array as large as the pool (its own offsets pass
    16 GiB)."""
    w = make_workload(seed=66, name="x", seq_lens=[333, 17, 64], q_lens=[1, 1, 1], num_q_heads=4, num_kv_heads=2,
                      head_size=128, block_size=16)
    print("large pool dequant", flush=True)
    d = _shifted(w)
    d.append_all()
    ok, ov = d.dequant()
    torch.cuda.synchronize()
    _check_writes(d, w)
    ref_pool = oracle_pool(w)
    rk, rv = O.dequant_paged(ref_pool, w.block_table, w.seq_lens, w.k_scale, w.v_scale, w.head_size)
    assert np.array_equal(bf16_to_np(ok), rk)
    assert np.array_equal(bf16_to_np(ov), rv)
    nb_all = int(d.pool.shape[0])
    out = torch.empty((nb_all, 2, w.block_size, w.num_kv_heads, w.head_size), dtype=torch.bfloat16, device="cuda")
    ids = (np.arange(w.num_blocks, dtype=np.int64) + d.shift).astype(np.int32)
    nvk.dequant_pages(d.pool, torch.from_numpy(ids).cuda(), d.k_scale, d.v_scale, out)
    torch.cuda.synchronize()
    got = bf16_to_np(out[d.shift:])
    del out
    assert np.array_equal(got, O.dequant_pages(ref_pool, np.arange(w.num_blocks), w.k_scale, w.v_scale,
                                               w.head_size))


@pytest.mark.parametrize("path", ["decode", "prefill_split"])
def test_large_pool_fp8_e4m3(path):
    kv = "fp8_e4m3"
    w = _fp8(_decode_case("split_d128") if path == "decode" else PREFILL["d128"](), kv)
    print(f"large pool fp8 {path}", flush=True)
    d = _shifted(w, kv)
    d.append_all()
    out = d.decode() if path == "decode" else d.prefill(causal=True, split=True)
    torch.cuda.synchronize()
    _check_writes(d, w, kv)
    ref = O.paged_attention(oracle_pool(w, kv), w.query, w.cu_q, w.block_table, w.seq_lens, w.k_scale,
                            w.v_scale, np.float32(d.sm_scale), w.head_size, causal=True, kv_dtype=kv)
    assert_attn_close(out, ref, f"large pool fp8 {path}")
