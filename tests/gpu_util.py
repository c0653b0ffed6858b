"""Helpers for the GPU parity tests: move a seeded workload to the device,
run the library through its binding, and build the oracle's view of the same
inputs. Expected values come only from the oracle."""
from __future__ import annotations

import math

import numpy as np
import torch

import bit_quantized_paged_amd as nvk
from oracle import nvfp4_oracle as O

# elementwise attention bound: |gpu - ref| <= ATOL + RTOL * |ref|
ATOL = 2e-3
RTOL = 1e-2


def bf16_dev(bits: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)


def i32_dev(x, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).to(device)


def i64_dev(x, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.int64)).to(device)


def scale_dev(s, device="cuda") -> torch.Tensor:
    return torch.tensor([float(np.float32(s))], dtype=torch.float32, device=device)


class Dev:
    """Device copies of a workload's inputs plus a pool of the chosen layout."""

    def __init__(self, w, layout="HND", device="cuda", kv_dtype="nvfp4"):
        self.w = w
        self.kv_dtype = kv_dtype
        self.pool = nvk.alloc_pool(w.num_blocks, w.block_size, w.num_kv_heads, w.head_size, layout, device,
                                   kv_dtype=kv_dtype)
        self.key = bf16_dev(w.key, device)
        self.value = bf16_dev(w.value, device)
        self.slots = i64_dev(w.slot_mapping, device)
        self.query = bf16_dev(w.query, device)
        self.bt = i32_dev(w.block_table, device)
        self.seq_lens = i32_dev(w.seq_lens, device)
        self.cu_q = i32_dev(w.cu_q, device)
        self.k_scale = scale_dev(w.k_scale, device)
        self.v_scale = scale_dev(w.v_scale, device)
        self.sm_scale = 1.0 / math.sqrt(w.head_size)

    def append_all(self):
        nvk.append(self.pool, self.key, self.value, self.slots, self.k_scale, self.v_scale)

    def pool_logical(self) -> np.ndarray:
        """The pool's bytes in logical order (any format, as uint8)."""
        return self.pool.contiguous().view(torch.uint8).cpu().numpy()

    def decode(self, q=None, max_seq_len=None, ws=None):
        """Decode over the whole batch. max_seq_len defaults to the longest
        sequence (0 lets the library bound lengths by the block table)."""
        w = self.w
        q = self.query if q is None else q
        out = torch.empty((w.num_seqs, w.num_q_heads, w.head_size), dtype=torch.bfloat16, device=q.device)
        if ws is None:
            ws = torch.zeros(nvk.decode_workspace_size(w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_size),
                             dtype=torch.uint8, device=q.device)
        msl = int(w.seq_lens.max(initial=0)) if max_seq_len is None else max_seq_len
        nvk.paged_attention_decode(self.pool, q, self.bt, self.seq_lens, msl, self.k_scale, self.v_scale,
                                   self.sm_scale, out, ws)
        return out

    def prefill_ws(self):
        """A zero-filled key-split workspace for this head size (one per Dev)."""
        if getattr(self, "_pws", None) is None:
            self._pws = torch.zeros(nvk.prefill_workspace_size(self.w.head_size), dtype=torch.uint8,
                                    device=self.query.device)
        return self._pws

    def prefill(self, causal=True, o_scale=None, split=False):
        """bf16 output, or FP8-E4M3 codes (uint8) with an output scale; with
        split, through the key split (the Dev's workspace)."""
        w = self.w
        out = torch.empty((int(w.cu_q[-1]), w.num_q_heads, w.head_size),
                          dtype=torch.bfloat16 if o_scale is None else torch.uint8, device=self.query.device)
        os_t = None if o_scale is None else torch.tensor([o_scale], dtype=torch.float32, device=self.query.device)
        nvk.paged_attention_prefill(self.pool, self.query, self.cu_q, int(w.q_lens.max(initial=0)), self.bt,
                                    self.seq_lens, int(w.seq_lens.max(initial=0)), self.k_scale, self.v_scale,
                                    self.sm_scale, out, causal=causal, o_scale=os_t,
                                    workspace=self.prefill_ws() if split else None)
        return out

    def dequant(self):
        w = self.w
        cu = np.zeros(w.num_seqs, np.int32)
        cu[1:] = np.cumsum(w.seq_lens)[:-1]
        rows = int(w.seq_lens.sum())
        ok = torch.zeros((rows, w.num_kv_heads, w.head_size), dtype=torch.bfloat16, device=self.pool.device)
        ov = torch.zeros_like(ok)
        nvk.dequant_paged(self.pool, self.bt, self.seq_lens, i32_dev(cu, self.pool.device),
                          int(w.seq_lens.max(initial=0)), self.k_scale, self.v_scale, ok, ov)
        return ok, ov


def oracle_pool(w, kv_dtype="nvfp4") -> np.ndarray:
    pool = np.zeros(O.pool_shape(w.num_blocks, w.block_size, w.num_kv_heads, w.head_size, kv_dtype), np.uint8)
    O.append(pool, w.key, w.value, w.slot_mapping, w.k_scale, w.v_scale, kv_dtype)
    return pool


def bf16_to_np(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def assert_attn_close(got: torch.Tensor, ref: np.ndarray, what=""):
    g = got.float().cpu().numpy().astype(np.float64)
    assert g.shape == ref.shape, (g.shape, ref.shape)
    assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    err = np.abs(g - ref)
    bound = ATOL + RTOL * np.abs(ref)
    worst = np.unravel_index(np.argmax(err / bound), err.shape)
    assert np.all(err <= bound), (f"{what}: max|err|={err.max():.3e} worst at {worst}: got {g[worst]:.6f} "
                                  f"ref {ref[worst]:.6f} ({(err <= bound).mean() * 100:.3f}% in band)")
    return float(err.max())


def fp8_out_bound(got, ref, os):
    """Largest |got - ref| a correct FP8 output can show.

    The kernel's fp32 result y satisfies |y - ref| <= 2e-3 + 1e-2 |ref| (the
    attention tolerance), and its code is E4M3 RNE of y / os, so the decoded
    value got differs from y by at most half the E4M3 step of y's binade
    (os times 2^(e - 3) for |y / os| in [2^e, 2^(e+1)), e >= -6; 2^-9 below
    2^-6). Rounding to nearest either stays in y's binade or carries into the
    next one up, never down, so the step at got's binade is at least the
    step at y's and the bound needs no knowledge of y:
    |got - ref| <= step(got) / 2 + 2e-3 + 1e-2 |ref|.
    """
    a = np.abs(got) / os
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -6)))
    step = 2.0 ** (e - 3) * os
    return step / 2 + 2e-3 + 1e-2 * np.abs(ref)
