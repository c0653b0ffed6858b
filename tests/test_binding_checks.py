"""The Python binding rejects mis-sized tensors before anything reaches the
C ABI, which sees only pointers: a wrong size there would be an
out-of-bounds device access. These run on the CPU with CPU tensors; a
correctly sized CPU tensor gets as far as the device check, so every case
below raises before any library call is made."""
import pytest
import torch

import bit_quantized_paged_amd as nvk

NB, BS, HKV, D, HQ = 6, 16, 2, 64, 4
FD = D // 2 + D // 16


def pool():
    return torch.zeros((NB, 2, HKV, BS, FD), dtype=torch.uint8).permute(0, 1, 3, 2, 4)


def scal(n=1, dt=torch.float32):
    return torch.ones(n, dtype=dt)


def kv(n=5, h=HKV, d=D):
    return torch.zeros((n, h, d), dtype=torch.bfloat16)


def raises(match, fn, *a, **k):
    with pytest.raises(ValueError, match=match):
        fn(*a, **k)


def test_append_rejects_mis_sized_inputs():
    p = pool()
    slots = torch.arange(5, dtype=torch.int64)
    raises("value must have shape", nvk.append, p, kv(5), kv(4), slots, scal(), scal())
    raises("key must have shape", nvk.append, p, kv(5, h=HKV + 1), kv(5, h=HKV + 1), slots, scal(), scal())
    raises("key must have shape", nvk.append, p, kv(5, d=128), kv(5, d=128), slots, scal(), scal())
    raises("slot_mapping must be 1-D with at least 5", nvk.append, p, kv(5), kv(5), slots[:4], scal(), scal())
    raises("slot_mapping must be torch.int64", nvk.append, p, kv(5), kv(5), slots.int(), scal(), scal())
    raises("k_scale must hold one", nvk.append, p, kv(5), kv(5), slots, scal(0), scal())
    raises("v_scale must be torch.float32", nvk.append, p, kv(5), kv(5), slots, scal(), scal(dt=torch.float64))
    raises("must be a device tensor", nvk.append, p, kv(5), kv(5), slots, scal(), scal())


def test_pool_descriptor_checks():
    raises("pool dtype", nvk.append, pool().float(), kv(5), kv(5), torch.arange(5), scal(), scal())
    bad = torch.zeros((NB, 2, BS, HKV, FD + 1), dtype=torch.uint8)
    raises("packed NVFP4 row width", nvk.append, bad, kv(5), kv(5), torch.arange(5), scal(), scal())
    raises("num_blocks, 2, block_size", nvk.append, torch.zeros((NB, 3, BS, HKV, FD), dtype=torch.uint8), kv(5),
           kv(5), torch.arange(5), scal(), scal())


def decode_args(B=3, maxb=4):
    return dict(pool=pool(), q=torch.zeros((B, HQ, D), dtype=torch.bfloat16),
                block_table=torch.zeros((B, maxb), dtype=torch.int32), seq_lens=torch.ones(B, dtype=torch.int32),
                max_seq_len=1, k_scale=scal(), v_scale=scal(), sm_scale=0.125,
                out=torch.zeros((B, HQ, D), dtype=torch.bfloat16), workspace=torch.zeros(64, dtype=torch.uint8))


def test_decode_rejects_mis_sized_inputs():
    a = decode_args()
    raises("out must have shape", nvk.paged_attention_decode, **{**a, "out": torch.zeros((3, HQ, D - 8),
                                                                                         dtype=torch.bfloat16)})
    raises("out must have shape", nvk.paged_attention_decode, **{**a, "out": torch.zeros((2, HQ, D),
                                                                                         dtype=torch.bfloat16)})
    raises("q must be", nvk.paged_attention_decode, **{**a, "q": torch.zeros((3, HQ, 128), dtype=torch.bfloat16)})
    raises("q must be", nvk.paged_attention_decode, **{**a, "q": torch.zeros((3, 3, D), dtype=torch.bfloat16)})
    raises("one row per sequence", nvk.paged_attention_decode,
           **{**a, "q": torch.zeros((4, HQ, D), dtype=torch.bfloat16),
              "out": torch.zeros((4, HQ, D), dtype=torch.bfloat16)})
    raises("block_table must be", nvk.paged_attention_decode,
           **{**a, "block_table": torch.zeros((2, 4), dtype=torch.int32)})
    raises("seq_lens must have shape", nvk.paged_attention_decode,
           **{**a, "seq_lens": torch.ones((3, 1), dtype=torch.int32)})
    raises("workspace must be torch.uint8", nvk.paged_attention_decode,
           **{**a, "workspace": torch.zeros(64, dtype=torch.int32)})
    # FP8 output: uint8 codes of q's shape, with a float32 output scale
    raises("out must be torch.uint8", nvk.paged_attention_decode, **{**a, "o_scale": scal()})
    raises("o_scale must hold one", nvk.paged_attention_decode,
           **{**a, "out": torch.zeros((3, HQ, D), dtype=torch.uint8), "o_scale": scal(0)})
    raises("must be a device tensor", nvk.paged_attention_decode, **a)


def test_prefill_rejects_mis_sized_inputs():
    B, T = 2, 7
    a = dict(pool=pool(), q=torch.zeros((T, HQ, D), dtype=torch.bfloat16),
             cu_seqlens_q=torch.tensor([0, 3, 7], dtype=torch.int32), max_q_len=4,
             block_table=torch.zeros((B, 4), dtype=torch.int32), seq_lens=torch.full((B,), 9, dtype=torch.int32),
             max_seq_len=9, k_scale=scal(), v_scale=scal(), sm_scale=0.125,
             out=torch.zeros((T, HQ, D), dtype=torch.bfloat16))
    raises("cu_seqlens_q must have shape", nvk.paged_attention_prefill,
           **{**a, "cu_seqlens_q": torch.tensor([0, 7], dtype=torch.int32)})
    raises("out must have shape", nvk.paged_attention_prefill,
           **{**a, "out": torch.zeros((T - 1, HQ, D), dtype=torch.bfloat16)})
    raises("q must be", nvk.paged_attention_prefill,
           **{**a, "q": torch.zeros((T, 5, D), dtype=torch.bfloat16), "out": torch.zeros((T, 5, D),
                                                                                         dtype=torch.bfloat16)})
    raises("block_table must be", nvk.paged_attention_prefill,
           **{**a, "block_table": torch.zeros((1, 4), dtype=torch.int32)})
    raises("must be a device tensor", nvk.paged_attention_prefill, **a)


def test_dequant_rejects_mis_sized_outputs():
    B = 2
    a = dict(pool=pool(), block_table=torch.zeros((B, 4), dtype=torch.int32), seq_lens=torch.ones(B, dtype=torch.int32),
             cu_seqlens_out=torch.tensor([0, 1], dtype=torch.int32), max_seq_len=1, k_scale=scal(), v_scale=scal(),
             out_key=kv(2), out_value=kv(2))
    raises("cu_seqlens_out must have shape", nvk.dequant_paged,
           **{**a, "cu_seqlens_out": torch.tensor([0, 1, 2], dtype=torch.int32)})
    raises("out_value must have shape", nvk.dequant_paged, **{**a, "out_value": kv(3)})
    raises("out_key must have shape", nvk.dequant_paged, **{**a, "out_key": kv(2, d=128), "out_value": kv(2, d=128)})
    raises("must be a device tensor", nvk.dequant_paged, **a)
    out = torch.zeros((NB, 2, BS, HKV, D), dtype=torch.bfloat16)
    raises("out must have shape", nvk.dequant_pages, pool(), None, scal(), scal(), out[:, :, :8])
    raises("page_ids must be 1-D", nvk.dequant_pages, pool(), torch.zeros((2, 2), dtype=torch.int32), scal(),
           scal(), out)


def test_codec_entry_points_reject_mis_sized_inputs():
    raises("value must have shape", nvk.qdq, kv(4), kv(5), scal(), scal())
    raises("out must have shape", nvk.fp8_to_bf16, torch.zeros(16, dtype=torch.uint8), scal(),
           torch.zeros(8, dtype=torch.bfloat16))
    raises("codes must have shape", nvk.quant_activations, torch.zeros((4, 32), dtype=torch.bfloat16), scal(),
           True, torch.zeros((4, 15), dtype=torch.uint8), torch.zeros(512, dtype=torch.uint8))
