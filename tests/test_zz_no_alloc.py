"""The allocation-free decode entry point, nvfp4_paged_attention_decode_noalloc,
called through the C ABI: its split-K scratch is the library's own device
array, shared by every call on the GPU. Calls in a row with different
batches and head geometries (the second smaller than the first, the third
the first again) must give the bits of nvfp4_paged_attention_decode with a
workspace, and the oracle's attention within the parity bound."""
import ctypes

import numpy as np
import pytest
import torch

import bit_quantized_paged_amd as nvk
from oracle import nvfp4_oracle as O
from workloads import make_workload
from gpu_util import Dev, assert_attn_close, oracle_pool


def _noalloc(lib, desc, q, q_st, q_sh, hq, bt, max_blocks, sl, B, max_seq_len, ks, vs, sm, out, stream):
    """One call of the C entry point; pointers are ints (device addresses)."""
    v = ctypes.c_void_p
    return lib.nvfp4_paged_attention_decode_noalloc(ctypes.byref(desc), v(q), q_st, q_sh, hq, v(bt), max_blocks,
                                                    v(sl), B, max_seq_len, v(ks), v(vs), ctypes.c_float(sm), v(out),
                                                    v(stream))


@pytest.mark.gpu
def test_noalloc_decode_matches_workspace_decode_in_a_row():
    cases = [
        # long sequences: split-K with partials and last-arrival combines (GQA 4, D = 128)
        make_workload(seed=71, name="x", seq_lens=[3000, 1, 2047, 900, 4500, 64], q_lens=[1] * 6, num_q_heads=32,
                      num_kv_heads=8, head_size=128, block_size=16),
        # smaller batch, other geometry (GQA 8, D = 256, 2 kv heads): the counters are where they were
        make_workload(seed=72, name="x", seq_lens=[700, 2500, 33], q_lens=[1] * 3, num_q_heads=16, num_kv_heads=2,
                      head_size=256, block_size=16),
    ]
    lib = nvk.library()
    for k, w in enumerate(cases + cases[:1]):
        print(f"no-alloc decode call {k}: {w.num_seqs} seqs, D={w.head_size}, Hkv={w.num_kv_heads}", flush=True)
        d = Dev(w, "HND")
        d.append_all()
        assert nvk.decode_plan(w.num_seqs, w.num_kv_heads, w.head_size, w.block_size, w.block_table.shape[1],
                               int(w.seq_lens.max())) == nvk.DECODE_SPLIT_K
        want = d.decode()
        out = torch.full_like(want, float("nan"))
        q = d.query
        st = _noalloc(lib, nvk._desc(d.pool), q.data_ptr(), q.stride(0), q.stride(1), q.shape[1], d.bt.data_ptr(),
                      d.bt.shape[1], d.seq_lens.data_ptr(), w.num_seqs, int(w.seq_lens.max()), d.k_scale.data_ptr(),
                      d.v_scale.data_ptr(), d.sm_scale, out.data_ptr(), torch.cuda.current_stream().cuda_stream)
        assert st == 0, lib.nvfp4kv_last_error()
        torch.cuda.synchronize()
        assert torch.equal(out, want), f"call {k}: differs from the workspace entry point"
        ref = O.paged_attention(oracle_pool(w), w.query, w.cu_q, w.block_table, w.seq_lens, w.k_scale, w.v_scale,
                                np.float32(d.sm_scale), w.head_size)
        assert_attn_close(out, ref, f"no-alloc decode call {k}")


def test_noalloc_decode_refuses_batches_beyond_its_scratch():
    """Refused on the host with WORKSPACE_TOO_SMALL before anything touches
    a device: partials beyond the 32 MiB array, or more (sequence, kv head)
    counters than it holds."""
    lib = nvk.library()
    fake = 1 << 20  # aligned placeholder pointers: nothing is dereferenced on these paths
    big = nvk.CacheDesc(fake, 1 << 16, 16, 16, 128, 0, 2 * 16 * 16 * 72, 16 * 16 * 72, 72, 16 * 72)
    assert _noalloc(lib, big, fake, 256 * 128, 128, 256, fake, 64, fake, 2000, 1024, fake, fake, 0.1, fake, 0) == 3
    assert b"decode scratch" in lib.nvfp4kv_last_error()
    many = nvk.CacheDesc(fake, 1 << 16, 16, 32, 64, 0, 2 * 32 * 16 * 36, 32 * 16 * 36, 36, 16 * 36)
    assert _noalloc(lib, many, fake, 32 * 64, 64, 32, fake, 4, fake, 4096, 64, fake, fake, 0.1, fake, 0) == 3
    assert b"split counters" in lib.nvfp4kv_last_error()
