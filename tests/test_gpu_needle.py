"""Needle recall through the quantised pages [RFC47684 "Verification": a
roughly 2K-token prompt whose answer sits at one position must be recalled
when the cache is NVFP4]. Each sequence of about 2K keys holds one key
aligned with its queries at a seeded position (page edges included) and a
distinct value there; attention must put nearly all its mass on that slot,
through decode (split-K) and through chunked prefill, and match the oracle
on the same quantised cache."""
import math

import numpy as np
import pytest
import torch

import bit_quantized_paged_amd as nvk
from oracle import nvfp4_oracle as O
from workloads import make_workload
from gpu_util import Dev, assert_attn_close, bf16_to_np, oracle_pool

pytestmark = pytest.mark.gpu

HQ, HKV, D, BS = 8, 2, 128, 16


def needle_workload(seed, lens, positions, q_lens=None):
    """Keys and values N(0, 1); in sequence b, at key positions[b], the key of
    kv head h is 2.5 x the shared query direction u_h of that head's query
    group and the value is 4 in every channel, so the needle's score is about
    2.5 |u|^2 / sqrt(D) ~ 28 against O(1) for the other keys."""
    q_lens = [1] * len(lens) if q_lens is None else q_lens
    w = make_workload(seed=seed, name="needle", seq_lens=lens, q_lens=q_lens, num_q_heads=HQ, num_kv_heads=HKV,
                      head_size=D, block_size=BS)
    rng = np.random.default_rng(seed + 1000)
    grp = HQ // HKV
    f = lambda bits: O.bf16_to_f32(bits)
    key, value, query = f(w.key).copy(), f(w.value).copy(), f(w.query).copy()
    for b, p in enumerate(positions):
        u = rng.standard_normal((HKV, D)).astype(np.float32)
        t = int(w.token_offsets[b]) + p
        key[t] = 2.5 * u
        value[t] = 4.0
        for h in range(HQ):
            query[int(w.cu_q[b]):int(w.cu_q[b + 1]), h] = u[h // grp]
    w.key, w.value, w.query = O.f32_to_bf16(key), O.f32_to_bf16(value), O.f32_to_bf16(query)
    amax = lambda x: np.float32(np.max(np.abs(O.bf16_to_f32(x))))
    w.k_scale = np.float32(amax(w.key) / np.float32(6 * 448))
    w.v_scale = np.float32(amax(w.value) / np.float32(6 * 448))
    return w


def test_needle_recall_decode_and_prefill():
    rng = np.random.default_rng(90)
    lens = [2048, 2000, 2048, 1999, 2048]
    positions = [0, 15, 16, 1998, int(rng.integers(0, 2048))]
    w = needle_workload(91, lens, positions)
    d = Dev(w, "HND")
    d.append_all()
    assert nvk.decode_plan(w.num_seqs, HKV, D, BS, w.block_table.shape[1], max(lens)) == nvk.DECODE_SPLIT_K
    out_d = d.decode()
    out_p = d.prefill()
    torch.cuda.synchronize()
    ref_pool = oracle_pool(w)
    ref = O.paged_attention(ref_pool, w.query, w.cu_q, w.block_table, w.seq_lens, w.k_scale, w.v_scale,
                            np.float32(1 / math.sqrt(D)), D)
    assert_attn_close(out_d, ref, "needle decode")
    assert_attn_close(out_p, ref, "needle prefill")
    # the needle's dequantised value row, and the attention mass it receives:
    # out = m * v_needle + (1 - m) * (mean of the others), the others' values
    # being O(1) noise, so |out - v_needle| <= (1 - m) * (4 + max|others|)
    _, vd = O.dequant_paged(ref_pool, w.block_table, w.seq_lens, w.k_scale, w.v_scale, D)
    vf = O.bf16_to_f32(vd).astype(np.float64)
    off = np.concatenate([[0], np.cumsum(w.seq_lens)])
    for b, p in enumerate(positions):
        vn = vf[off[b] + p]                       # [HKV, D]
        others = np.delete(vf[off[b]:off[b + 1]], p, axis=0)
        spread = 4.0 + np.max(np.abs(others))
        for out, path in ((out_d, "decode"), (out_p, "prefill")):
            g = out[b].float().cpu().numpy()
            for h in range(HQ):
                dev_ = np.max(np.abs(g[h] - vn[h // (HQ // HKV)]))
                mass = 1.0 - dev_ / spread
                assert mass > 0.99, f"{path} seq {b} needle at {p}, head {h}: mass >= {mass:.4f} only"


def test_needle_recall_in_a_long_chunk():
    """Chunked prefill of 256 queries over 2048 cached keys, with the needle in
    the cached prefix: every query row of the chunk recalls it."""
    w = needle_workload(92, [2304], [777], q_lens=[256])
    d = Dev(w, "HND")
    d.append_all()
    out = d.prefill()
    torch.cuda.synchronize()
    ref = O.paged_attention(oracle_pool(w), w.query, w.cu_q, w.block_table, w.seq_lens, w.k_scale, w.v_scale,
                            np.float32(1 / math.sqrt(D)), D)
    assert_attn_close(out, ref, "needle in a 256-query chunk")
    _, vd = O.dequant_paged(oracle_pool(w), w.block_table, w.seq_lens, w.k_scale, w.v_scale, D)
    vn = O.bf16_to_f32(vd).astype(np.float64)[777]
    g = out.float().cpu().numpy()
    assert np.max(np.abs(g - vn[np.arange(HQ) // (HQ // HKV)][None])) < 0.05 * 4.0
