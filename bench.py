#!/usr/bin/env python3
"""Benchmark of the NVFP4 paged KV cache hot path on one MI355X.

A step is one serving pass over the batch: quantize-append every sequence's
new tokens into the pool (slot mapping), then paged attention over the
quantised cache (decode for 1-token sequences, chunked prefill for the
rest). K steps are captured into one HIP graph and timed as a whole; pool
copies rotate between steps so that no step finds its cache in the 256 MB
Infinity Cache (every copy holds identical bytes). Decode-only and
append-only graphs over the same rotation give the per-kernel times used for
the roofline, and a read-only stream of the same bytes over the same
rotation gives the read ceiling the decode stream is judged against.

The headline workload (default: the long-context decode batch, the largest
decode stream) is measured in full; the mixed serving batch's decode half
and prefill are measured beside it and reported as extra fields.

Prints one JSON line. `value` is the decode attention's effective HBM
bandwidth (cache bytes + q + out + block ids + lengths over the decode
kernel's time); append Mtokens/s and the other rates are extra fields.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_F16_PEAK_TFLOPS = 2500.0
MALL_BYTES = 256 << 20
WORKLOADS = {"tiny_decode": 1, "small_decode": 2, "long_decode": 3, "chunked_prefill": 4, "mixed_serving": 5}
SERVING_BATCH = "mixed_serving"
METRIC = "decode attention effective HBM GB/s (% of peak) + append Mtokens/s, NVFP4 KV"
KERNEL_SOURCES = ["bit_quantized_paged_amd/csrc/attn.hip", "bit_quantized_paged_amd/csrc/attn_core.hpp",
                  "bit_quantized_paged_amd/csrc/device_common.hpp"]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="long_decode", choices=sorted(WORKLOADS))
    ap.add_argument("--copies", type=int, default=0, help="pool copies to rotate (0: enough to exceed the MALL 3x)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--prefill-grid", action="store_true",
                    help="also time the prefill without the key split (one workgroup per job), as prefill_grid_us")
    ap.add_argument("--no-serving-batch", action="store_true",
                    help="skip the mixed serving batch measured beside the headline workload")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a 512 MiB device copy (to scale rocprofv3 FETCH_SIZE/WRITE_SIZE)")
    return ap.parse_args()


def source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def exact_decode(wd, sm_scale, dev):
    """fp32 softmax attention of each decode query over its sequence's
    unquantised bf16 keys and values (the accuracy yardstick for the cache
    formats; plain torch, not the oracle)."""
    import numpy as np
    import torch
    B, Hq, D = wd.query.shape
    Hkv = wd.key.shape[1]
    grp = Hq // Hkv
    f32 = lambda bits: torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16).float()
    q = f32(wd.query)
    out = torch.zeros((B, Hq, D), dtype=torch.float32, device=dev)
    for b in range(B):
        t0, t1 = int(wd.token_offsets[b]), int(wd.token_offsets[b + 1])
        if t1 == t0:
            continue
        k = f32(wd.key[t0:t1]).repeat_interleave(grp, dim=1).permute(1, 2, 0).contiguous()   # [Hq, D, L]
        v = f32(wd.value[t0:t1]).repeat_interleave(grp, dim=1).permute(1, 0, 2).contiguous()  # [Hq, L, D]
        p = torch.softmax(torch.bmm(q[b][:, None, :], k) * sm_scale, dim=-1)                   # [Hq, 1, L]
        out[b] = torch.bmm(p, v)[:, 0, :]
    return out


def read_traffic(kernel: str, workload: str):
    """HBM bytes per launch of a workload's main kernel from the committed
    counter summary, if it was taken on the current kernel sources (else None)."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.md")
    if not os.path.exists(path):
        return None
    rec = {}
    for line in open(path):
        if line.startswith("traffic:"):
            for kv in line[len("traffic:"):].split():
                k, v = kv.split("=")
                rec[k] = v
    if rec.get("source_hash") != source_hash():
        return None
    return float(rec["bytes_per_launch"])


class Timer:
    """Graph capture of K calls and replay timing on the current stream."""

    def __init__(self, K):
        import torch
        self.K = K
        self.cap_stream = torch.cuda.Stream()

    def capture(self, fn, n):
        """A graph of K calls fn(s % n)."""
        import torch
        g = torch.cuda.CUDAGraph()
        self.cap_stream.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(self.cap_stream):
            with torch.cuda.graph(g, stream=self.cap_stream):
                for s in range(self.K):
                    fn(s % n)
        torch.cuda.current_stream().wait_stream(self.cap_stream)
        return g

    def time(self, g, reps=1):
        """Seconds for one replay of g (K steps): the median of `reps` timed
        replays on the current stream (the stream the kernels run on), after
        untimed warm replays (the first replays on a fresh GPU run slower
        while its clocks ramp up)."""
        import torch
        for _ in range(3):
            g.replay()
        torch.cuda.synchronize()
        stream = torch.cuda.current_stream()
        gpu, wall = [], []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            e0.record(stream)
            g.replay()
            e1.record(stream)
            torch.cuda.synchronize()
            wall.append(time.perf_counter() - t0)
            gpu.append(e0.elapsed_time(e1) / 1e3)
        order = sorted(range(reps), key=lambda r: gpu[r])
        mid = order[reps // 2]
        return gpu[mid], wall[mid]

    def per_call(self, fn, n, reps=3):
        """Seconds per call of fn over a graph of K calls rotated over n."""
        g = self.capture(fn, n)
        t, _ = self.time(g, reps)
        del g
        return t / self.K


def run_workload(args, name, full, dev):
    """Time one workload's step and kernels. full: also the codec, FP8-cache,
    activation-quantisation and bulk-append measurements and the read-stream
    ceiling. Returns (results dict, workload, decode/prefill index arrays)."""
    import numpy as np
    import torch

    import bit_quantized_paged_amd as nvk
    from bit_quantized_paged_amd import probe
    from workloads import fp8_kv_scales, make_activations, make_config

    cfg = WORKLOADS[name]
    t_gen = time.perf_counter()
    w = make_config(cfg)
    gen_s = time.perf_counter() - t_gen
    B, Hq, Hkv, D, bs = w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_size, w.block_size
    fd = D // 2 + D // 16
    sm_scale = 1.0 / math.sqrt(D)
    K = args.steps
    T = Timer(K)

    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)
    i64 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int64)).to(dev)

    cached = w.cached_mask()
    new = ~cached
    k_scale = torch.tensor([float(w.k_scale)], device=dev)
    v_scale = torch.tensor([float(w.v_scale)], device=dev)

    # ---- pool copies, filled with the cached prefix (outside any timing)
    base = torch.zeros((w.num_blocks, 2, Hkv, bs, fd), dtype=torch.uint8, device=dev)
    pool0 = base.permute(0, 1, 3, 2, 4)
    if cached.any():
        kc, vc, sc = bf(w.key[cached]), bf(w.value[cached]), i64(w.slot_mapping[cached])
        nvk.append(pool0, kc, vc, sc, k_scale, v_scale)
        del kc, vc, sc
    pool_bytes = base.numel()
    copies = args.copies or max(2, math.ceil(3 * MALL_BYTES / pool_bytes))
    bases = [base] + [base.clone() for _ in range(copies - 1)]
    pools = [b_.permute(0, 1, 3, 2, 4) for b_ in bases]

    k_new, v_new, s_new = bf(w.key[new]), bf(w.value[new]), i64(w.slot_mapping[new])
    n_new = int(new.sum())

    dec_idx = np.nonzero(w.q_lens == 1)[0]
    pre_idx = np.nonzero(w.q_lens != 1)[0]
    wd = w.subset(dec_idx) if len(dec_idx) else None
    wp = w.subset(pre_idx) if len(pre_idx) else None
    if wd is not None:
        qd, btd, sld = bf(wd.query), i32(wd.block_table), i32(wd.seq_lens)
        outd = torch.empty((wd.num_seqs, Hq, D), dtype=torch.bfloat16, device=dev)
        wsd = torch.zeros(nvk.decode_workspace_size(wd.num_seqs, Hq, Hkv, D), dtype=torch.uint8, device=dev)
        maxd = int(wd.seq_lens.max())
    if wp is not None:
        qp, btp, slp, cup = bf(wp.query), i32(wp.block_table), i32(wp.seq_lens), i32(wp.cu_q)
        outp = torch.empty((int(wp.cu_q[-1]), Hq, D), dtype=torch.bfloat16, device=dev)
        outp_grid = torch.empty_like(outp)
        maxq, maxp = int(wp.q_lens.max()), int(wp.seq_lens.max())
        # the key split's workspace: zero-filled once, its counters are left
        # at zero by every call
        wsp = torch.zeros(nvk.prefill_workspace_size(D), dtype=torch.uint8, device=dev)

    def do_append(r):
        nvk.append(pools[r], k_new, v_new, s_new, k_scale, v_scale)

    def do_decode(r):
        nvk.paged_attention_decode(pools[r], qd, btd, sld, maxd, k_scale, v_scale, sm_scale, outd, wsd)

    def do_prefill(r):
        nvk.paged_attention_prefill(pools[r], qp, cup, maxq, btp, slp, maxp, k_scale, v_scale, sm_scale, outp,
                                    workspace=wsp)

    def do_prefill_grid(r):
        # one workgroup per job, no key split (reported beside it)
        nvk.paged_attention_prefill(pools[r], qp, cup, maxq, btp, slp, maxp, k_scale, v_scale, sm_scale, outp_grid)

    def step(r):
        do_append(r)
        if wd is not None:
            do_decode(r)
        if wp is not None:
            do_prefill(r)

    # ---- eager warmup, then a reference result for the graph check
    for s in range(args.warmup):
        step(s % copies)
    torch.cuda.synchronize()
    ref_d = outd.clone() if wd is not None else None
    ref_p = outp.clone() if wp is not None else None

    g_step = T.capture(step, copies)
    step_gpu_s, step_wall_s = T.time(g_step)
    del g_step
    if wd is not None:
        assert torch.equal(outd, ref_d), "graph replay of the step differs from the eager decode"
    if wp is not None:
        assert torch.equal(outp, ref_p), "graph replay of the step differs from the eager prefill"
    res = {"name": w.name, "seed": cfg, "gen_s": gen_s, "K": K, "copies": copies, "pool_bytes": pool_bytes,
           "step_gpu_s": step_gpu_s, "step_wall_s": step_wall_s, "n_new": n_new,
           "append_s": T.per_call(do_append, copies), "B": B, "Hq": Hq, "Hkv": Hkv, "D": D, "bs": bs,
           "total_tokens": int(w.seq_lens.sum()), "decode_seqs": int(len(dec_idx)), "prefill_seqs": int(len(pre_idx))}
    res["append_bytes"] = n_new * (Hkv * (2 * 2 * D + 2 * fd) + 8)
    extra = {}
    if wd is not None:
        res["decode_s"] = T.per_call(do_decode, copies)
        assert torch.equal(outd, ref_d), "graph replay of decode differs from eager"
        res["decode_bytes"] = (int(wd.seq_lens.astype(np.int64).sum()) * Hkv * 2 * fd + 2 * wd.num_seqs * Hq * D * 2
                               + 4 * int(np.sum((wd.seq_lens + bs - 1) // bs)) + 4 * wd.num_seqs)
        plan = nvk.decode_plan(wd.num_seqs, Hkv, D, bs, int(wd.block_table.shape[1]), maxd, "nvfp4")
        res["decode_kernel"] = "decode_pair_kernel" if plan == nvk.DECODE_PER_PAIR else "decode_split_kernel"
    if wp is not None:
        res["prefill_s"] = T.per_call(do_prefill, copies)
        assert torch.equal(outp, ref_p), "graph replay of prefill differs from eager"
        if args.prefill_grid:
            res["prefill_grid_s"] = T.per_call(do_prefill_grid, copies)
        pairs = 0
        for b in range(wp.num_seqs):
            L, q = int(wp.seq_lens[b]), int(wp.q_lens[b])
            pairs += q * (L - q) + q * (q + 1) // 2
        res["prefill_flops"] = 4.0 * D * Hq * pairs
        # every cached row of a prefill sequence once per kv head, the bf16
        # queries in and outputs out, the block ids and the per-sequence
        # lengths and offsets (the same accounting as the decode's)
        res["prefill_bytes"] = (int(wp.seq_lens.astype(np.int64).sum()) * Hkv * 2 * fd
                                + 2 * int(wp.q_lens.astype(np.int64).sum()) * Hq * D * 2
                                + 4 * int(np.sum((wp.seq_lens + bs - 1) // bs)) + 4 * (2 * wp.num_seqs + 1))
    if not full:
        return res, extra, w, dec_idx, pre_idx

    if wd is not None:
        # ---- read ceiling: a plain read-only stream of the decode's bytes
        # over the same pool rotation (each copy's first bytes, contiguous),
        # the fastest of a few grid sizes (one to eight workgroups per CU)
        nb = min(res["decode_bytes"], pool_bytes) // 16 * 16
        cus = torch.cuda.get_device_properties(dev).multi_processor_count
        sink = torch.zeros(4 * 8 * cus, dtype=torch.int32, device=dev)
        sweep = {}
        for per_cu in (1, 2, 4, 8):
            sweep[per_cu] = T.per_call(lambda r: probe.read_stream(bases[r], nb, sink, per_cu * cus), copies)
        best = min(sweep, key=sweep.get)
        extra["read_stream_ceiling_gbs"] = round(nb / sweep[best] / 1e9, 1)
        extra["read_stream_us"] = round(sweep[best] * 1e6, 2)
        extra["read_stream_bytes"] = nb
        extra["read_stream_sweep_us"] = {f"{k}_wg_per_cu": round(v * 1e6, 2) for k, v in sweep.items()}
        # ---- the same pages the decode reads, read as a plain gather through
        # its block table (every K and V slab of every page, whole last pages)
        gsweep = {}
        for per_cu in (2, 4, 6, 8):
            splits = max(1, per_cu * cus // (wd.num_seqs * Hkv))
            gsink = torch.zeros(4 * wd.num_seqs * Hkv * splits, dtype=torch.int32, device=dev)
            gsweep[per_cu] = T.per_call(lambda r: probe.read_pages(pools[r], btd, sld, gsink, splits), copies)
            del gsink
        gbest = min(gsweep, key=gsweep.get)
        pages = int(np.sum((wd.seq_lens + bs - 1) // bs))
        g_bytes = pages * Hkv * 2 * bs * fd
        extra["page_gather_us"] = round(gsweep[gbest] * 1e6, 2)
        extra["page_gather_gbs"] = round(g_bytes / gsweep[gbest] / 1e9, 1)
        extra["page_gather_bytes"] = g_bytes
        extra["page_gather_sweep_us"] = {f"{k}_wg_per_cu": round(v * 1e6, 2) for k, v in gsweep.items()}
        del sink

        # ---- paged dequantize of the decode batch (reported, not part of the step)
        rows = int(wd.seq_lens.sum())
        cu = np.zeros(wd.num_seqs, np.int32)
        cu[1:] = np.cumsum(wd.seq_lens)[:-1]
        cud = i32(cu)
        ok = torch.empty((rows, Hkv, D), dtype=torch.bfloat16, device=dev)
        ov = torch.empty_like(ok)
        deq_s = T.per_call(lambda r: nvk.dequant_paged(pools[r], btd, sld, cud, maxd, k_scale, v_scale, ok, ov),
                           copies)
        deq_bytes = rows * Hkv * 2 * (fd + 2 * D) + 4 * int(np.sum((wd.seq_lens + bs - 1) // bs))
        extra["dequant_gbs"] = round(deq_bytes / deq_s / 1e9, 1)
        extra["dequant_us"] = round(deq_s * 1e6, 2)
        del ok, ov

        # ---- page-form dequantize of the pages the decode batch uses
        used = np.unique(np.concatenate([wd.block_table[b, :(int(wd.seq_lens[b]) + bs - 1) // bs]
                                         for b in range(wd.num_seqs)])).astype(np.int32)
        ids = i32(used)
        pages_out = torch.empty((w.num_blocks, 2, bs, Hkv, D), dtype=torch.bfloat16, device=dev)
        pg_s = T.per_call(lambda r: nvk.dequant_pages(pools[r], ids, k_scale, v_scale, pages_out), copies)
        del pages_out
        pg_bytes = len(used) * 2 * bs * Hkv * (fd + 2 * D) + 4 * len(used)
        extra["dequant_pages_gbs"] = round(pg_bytes / pg_s / 1e9, 1)
        extra["dequant_pages_us"] = round(pg_s * 1e6, 2)

        # ---- FP8-E4M3 output (output scale 1) and its bf16 epilogue; the
        # extra rounding is measured against the bf16 output of the same decode
        o_s = torch.ones(1, dtype=torch.float32, device=dev)
        codes = torch.empty(outd.shape, dtype=torch.uint8, device=dev)
        f8_s = T.per_call(lambda r: nvk.paged_attention_decode(pools[r], qd, btd, sld, maxd, k_scale, v_scale,
                                                               sm_scale, codes, wsd, o_scale=o_s), copies)
        back = torch.empty_like(outd)
        ep_s = T.per_call(lambda r: nvk.fp8_to_bf16(codes, o_s, back), copies)
        torch.cuda.synchronize()
        ref16 = ref_d.float()
        diff = (back.float() - ref16).abs()
        rel = diff / ref16.abs().clamp_min(1e-2)
        extra["decode_fp8out_us"] = round(f8_s * 1e6, 2)
        extra["fp8_epilogue_us"] = round(ep_s * 1e6, 2)
        extra["fp8_out_extra_err"] = {"max_abs": round(float(diff.max()), 5),
                                      "rms_abs": round(float(diff.pow(2).mean().sqrt()), 6),
                                      "max_rel": round(float(rel.max()), 5), "ref": "bf16 output of the same decode"}
        del codes, back

    # ---- quantize-dequantize emulation in place on copies of the workload's
    # K/V, rotated so that no call finds its rows in the MALL
    kq, vq = bf(w.key), bf(w.value)
    q_copies = max(2, math.ceil(3 * MALL_BYTES / (2 * kq.numel() * 2)))
    kvs = [(kq, vq)] + [(kq.clone(), vq.clone()) for _ in range(q_copies - 1)]
    qdq_s = T.per_call(lambda r: nvk.qdq(kvs[r][0], kvs[r][1], k_scale, v_scale), q_copies)
    extra["qdq_gbs"] = round(2 * 2 * kq.numel() * 2 / qdq_s / 1e9, 1)
    extra["qdq_us"] = round(qdq_s * 1e6, 2)
    extra["qdq_tokens"] = int(kq.shape[0])
    del kq, vq, kvs

    # ---- activation quantisation with swizzled scales: the hidden states of a
    # 4 x 2048-token prefill chunk, hidden size 32 heads x 128, rotated past the MALL
    am, ak = 8192, 4096
    abits, ag = make_activations(seed=4, m=am, k=ak)
    a0 = torch.from_numpy(abits.view(np.int16)).to(dev).view(torch.bfloat16)
    a_copies = max(2, math.ceil(3 * MALL_BYTES / (am * ak * 2)))
    acts = [a0] + [a0.clone() for _ in range(a_copies - 1)]
    ags = torch.tensor([float(ag)], dtype=torch.float32, device=dev)
    a_codes, a_sf = nvk.quant_activations(a0, ags, True)
    aq_s = T.per_call(lambda r: nvk.quant_activations(acts[r], ags, True, a_codes, a_sf), a_copies)
    aq_bytes = am * ak * 2 + am * ak // 2 + a_sf.numel()
    extra["act_quant_us"] = round(aq_s * 1e6, 2)
    extra["act_quant_gbs"] = round(aq_bytes / aq_s / 1e9, 1)
    extra["act_quant_shape"] = [am, ak]
    del acts, a0, a_codes, a_sf

    # ---- the same decode and prefill over FP8 caches (E4M3, E5M2) of the same
    # K/V, with the per-tensor scale amax / largest finite value: the
    # kernel-level NVFP4-vs-FP8 comparison
    if wd is not None or wp is not None:
        exact = exact_decode(wd, sm_scale, dev) if wd is not None else None

        def err_vs_exact(o):
            e = (o.float() - exact).abs()
            return {"max_abs": round(float(e.max()), 5), "rms": round(float(e.pow(2).mean().sqrt()), 6)}

        if wd is not None:
            extra["nvfp4_decode_err_vs_exact"] = err_vs_exact(ref_d)
        fp8d, fp8p = {}, {}
        all_k, all_v, all_s = bf(w.key), bf(w.value), i64(w.slot_mapping)
        for kv in ("fp8_e4m3", "fp8_e5m2"):
            ks8, vs8 = fp8_kv_scales(w, kv)
            ks8_t = torch.tensor([float(ks8)], dtype=torch.float32, device=dev)
            vs8_t = torch.tensor([float(vs8)], dtype=torch.float32, device=dev)
            b8 = torch.zeros((w.num_blocks, 2, Hkv, bs, D), dtype=nvk.KV_DTYPES[kv][1], device=dev)
            nvk.append(b8.permute(0, 1, 3, 2, 4), all_k, all_v, all_s, ks8_t, vs8_t)
            n8 = max(2, math.ceil(3 * MALL_BYTES / b8.numel()))
            p8s = [b8.permute(0, 1, 3, 2, 4)] + [b8.clone().permute(0, 1, 3, 2, 4) for _ in range(n8 - 1)]
            if wd is not None:
                out8 = torch.empty_like(outd)
                t8 = T.per_call(lambda r: nvk.paged_attention_decode(p8s[r], qd, btd, sld, maxd, ks8_t, vs8_t,
                                                                     sm_scale, out8, wsd), n8)
                torch.cuda.synchronize()
                b8_bytes = (int(wd.seq_lens.astype(np.int64).sum()) * Hkv * 2 * D + 2 * wd.num_seqs * Hq * D * 2
                            + 4 * int(np.sum((wd.seq_lens + bs - 1) // bs)) + 4 * wd.num_seqs)
                plan8 = nvk.decode_plan(wd.num_seqs, Hkv, D, bs, int(wd.block_table.shape[1]), maxd, kv)
                fp8d[kv] = {"decode_us": round(t8 * 1e6, 2), "gbs": round(b8_bytes / t8 / 1e9, 1),
                            "cache_bytes_per_launch": b8_bytes, "pool_copies": n8,
                            "kernel": "decode_pair_kernel" if plan8 == nvk.DECODE_PER_PAIR else "decode_split_kernel",
                            "time_vs_nvfp4": round(t8 / res["decode_s"], 3), "err_vs_exact": err_vs_exact(out8)}
                del out8
            if wp is not None:
                outp8 = torch.empty_like(outp)
                t8 = T.per_call(lambda r: nvk.paged_attention_prefill(p8s[r], qp, cup, maxq, btp, slp, maxp, ks8_t,
                                                                      vs8_t, sm_scale, outp8, workspace=wsp), n8)
                fp8p[kv] = {"prefill_us": round(t8 * 1e6, 2), "time_vs_nvfp4": round(t8 / res["prefill_s"], 3)}
                del outp8
            del p8s, b8
        if fp8d:
            extra["fp8_kv_decode"] = fp8d
        if fp8p:
            extra["fp8_kv_prefill"] = fp8p
        del all_k, all_v, all_s

    # ---- bulk append: every cached token of the workload in one call (the
    # pool fill, K/V inputs rotated past the MALL)
    n_cached = int(cached.sum())
    if n_cached:
        kc, vc, sc = bf(w.key[cached]), bf(w.value[cached]), i64(w.slot_mapping[cached])
        kv_bytes = 2 * kc.numel() * 2
        b_copies = max(1, math.ceil(3 * MALL_BYTES / kv_bytes))
        kvc = [(kc, vc)] + [(kc.clone(), vc.clone()) for _ in range(b_copies - 1)]
        bulk_s = T.per_call(lambda r: nvk.append(pools[r % copies], kvc[r % b_copies][0], kvc[r % b_copies][1], sc,
                                                 k_scale, v_scale), copies * b_copies)
        del kvc, kc, vc, sc
        bulk_bytes = n_cached * (Hkv * (2 * 2 * D + 2 * fd) + 8)
        extra["bulk_append_tokens"] = n_cached
        extra["bulk_append_us"] = round(bulk_s * 1e6, 2)
        extra["bulk_append_mtok_s"] = round(n_cached / bulk_s / 1e6, 1)
        extra["bulk_append_gbs"] = round(bulk_bytes / bulk_s / 1e9, 1)

    # ---- device-copy ceiling (1 GiB read + write), for reference
    csrc_t = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    cdst_t = torch.empty_like(csrc_t)
    for _ in range(3):
        cdst_t.copy_(csrc_t)
    torch.cuda.synchronize()
    ct = []
    for _ in range(5):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        cdst_t.copy_(csrc_t)
        e1.record()
        torch.cuda.synchronize()
        ct.append(e0.elapsed_time(e1) / 1e3)
    extra["device_copy_ceiling_gbs"] = round(2 * csrc_t.numel() / sorted(ct)[2] / 1e9, 1)
    del csrc_t, cdst_t
    return res, extra, w, dec_idx, pre_idx


def rates(res):
    """Per-launch rates of one workload's kernels."""
    out = {"append_us": round(res["append_s"] * 1e6, 2),
           "append_mtok_s": round(res["n_new"] / res["append_s"] / 1e6, 3),
           "append_gbs": round(res["append_bytes"] / res["append_s"] / 1e9, 1),
           "step_gpu_us": round(res["step_gpu_s"] / res["K"] * 1e6, 2)}
    if "decode_s" in res:
        gbs = res["decode_bytes"] / res["decode_s"] / 1e9
        out.update({"decode_us": round(res["decode_s"] * 1e6, 2), "decode_gbs": round(gbs, 1),
                    "decode_pct_of_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 1), "decode_bytes": res["decode_bytes"],
                    "decode_kernel": res["decode_kernel"]})
    if "prefill_s" in res:
        tf = res["prefill_flops"] / res["prefill_s"] / 1e12
        out.update({"prefill_us": round(res["prefill_s"] * 1e6, 2), "prefill_tflops": round(tf, 2),
                    "prefill_pct_of_mfma_peak": round(100 * tf / MFMA_F16_PEAK_TFLOPS, 2),
                    "prefill_bytes": res["prefill_bytes"],
                    "prefill_kernel": "prefill_plan_kernel + prefill_kernel (key split)"})
        if "prefill_grid_s" in res:
            out["prefill_grid_us"] = round(res["prefill_grid_s"] * 1e6, 2)
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: --gpus {args.gpus} is not supported (the NVFP4 KV path here is "
              "single-GPU; see the design notes for how it would shard)", file=sys.stderr)
        sys.exit(2)

    import torch

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.calibrate_copy:
        src = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": src.numel()}))
        return

    res, extra, w, dec_idx, pre_idx = run_workload(args, args.workload, True, dev)
    r = rates(res)
    K = args.steps
    out = {"metric": METRIC, "unit": "GB/s", "n_gpus": 1, "steps": K, "warmup": args.warmup,
           "ms_per_step": round(res["step_wall_s"] / K * 1e3, 5), "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "f16", "data": "synthetic"}
    roof = None
    if "decode_s" in res:
        out["value"] = r["decode_gbs"]
        roof = {"bound": "hbm", "achieved": r["decode_gbs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(r["decode_gbs"] / HBM_PEAK_GBS, 4),
                "traffic": read_traffic(res["decode_kernel"], res["name"]), "kernel": res["decode_kernel"],
                "bytes_per_launch": res["decode_bytes"], "avg_launch_us": round(res["decode_s"] * 1e6, 3)}
        if "read_stream_ceiling_gbs" in extra:
            # ceilings measured in the same run: a contiguous read of the
            # decode's byte count, and a plain gather of the decode's own pages
            # (time ratio: that gather's time over the decode's)
            roof["read_stream_ceiling_gbs"] = extra["read_stream_ceiling_gbs"]
            roof["frac_of_read_stream_ceiling"] = round(r["decode_gbs"] / extra["read_stream_ceiling_gbs"], 4)
            roof["page_gather_us"] = extra["page_gather_us"]
            roof["frac_of_page_gather_time"] = round(extra["page_gather_us"] / r["decode_us"], 4)
    elif "prefill_s" in res:
        out["value"] = r["prefill_tflops"]
        out["unit"] = "TFLOP/s"
        roof = {"bound": "mfma", "achieved": r["prefill_tflops"], "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(r["prefill_tflops"] / MFMA_F16_PEAK_TFLOPS, 4),
                "traffic": read_traffic("prefill_kernel", res["name"]), "bytes_per_launch": res["prefill_bytes"],
                "kernel": "prefill_kernel", "flops_per_launch": res["prefill_flops"],
                "avg_launch_us": round(res["prefill_s"] * 1e6, 3)}
    out["config"] = {"workload": res["name"], "num_seqs": res["B"], "num_q_heads": res["Hq"],
                     "num_kv_heads": res["Hkv"], "head_dim": res["D"], "block_size": res["bs"],
                     "total_tokens": res["total_tokens"], "new_tokens": res["n_new"],
                     "decode_seqs": res["decode_seqs"], "prefill_seqs": res["prefill_seqs"], "kv_dtype": "nvfp4",
                     "pool_copies": res["copies"], "pool_bytes": res["pool_bytes"], "seed": res["seed"]}
    out["roofline"] = roof
    out.update(r)
    out.update(extra)
    out["source_hash"] = source_hash()
    out["input_gen_s"] = round(res["gen_s"], 2)

    if not args.no_serving_batch and args.workload != SERVING_BATCH:
        # the mixed serving batch beside the headline: its decode half and its
        # prefill, each timed as above (extra fields only)
        torch.cuda.empty_cache()
        sres, _, _, _, _ = run_workload(args, SERVING_BATCH, False, dev)
        sr = rates(sres)
        out["serving_batch"] = {"workload": sres["name"], "decode_seqs": sres["decode_seqs"],
                                "prefill_seqs": sres["prefill_seqs"], **sr}
        torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, dec_idx, pre_idx, 1.0 / math.sqrt(w.head_size))
    print(json.dumps(out), flush=True)


def cpu_baseline(w, dec_idx, pre_idx, sm_scale):
    """The oracle, untuned, on a bounded sample of the same step: quantize-
    append of the sampled sequences' new tokens, then their attention. The
    cached prefix of the sample is quantised beforehand (not timed). `cores`
    is the most threads the oracle can use: its matrix products run on the
    BLAS thread pool, its elementwise NumPy work on one thread."""
    import numpy as np
    import torch
    from oracle import nvfp4_oracle as O
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas_threads = 1
    # sample: whole sequences, decode ones first, up to ~300k (token, kv head) rows
    order = list(dec_idx) + list(pre_idx)
    budget, picked = 300_000, []
    for b in order:
        if picked and sum(int(w.seq_lens[x]) for x in picked) * w.num_kv_heads + int(w.seq_lens[b]) * w.num_kv_heads > budget:
            break
        picked.append(b)
    ws = w.subset(np.array(picked))
    cm = ws.cached_mask()
    pool = np.zeros(O.pool_shape(ws.num_blocks, ws.block_size, ws.num_kv_heads, ws.head_size), np.uint8)
    O.append(pool, ws.key[cm], ws.value[cm], ws.slot_mapping[cm], ws.k_scale, ws.v_scale)
    fd = ws.full_dim
    t0 = time.perf_counter()
    reps = 0
    while True:
        O.append(pool, ws.key[~cm], ws.value[~cm], ws.slot_mapping[~cm], ws.k_scale, ws.v_scale)
        O.paged_attention(pool, ws.query, ws.cu_q, ws.block_table, ws.seq_lens, ws.k_scale, ws.v_scale,
                          np.float32(sm_scale), ws.head_size)
        reps += 1
        el = time.perf_counter() - t0
        if el >= 10.0 or reps >= 20:
            break
    per = el / reps
    dec_bytes = int(ws.seq_lens.astype(np.int64).sum()) * ws.num_kv_heads * 2 * fd
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        affinity = None
    return {"value": round(dec_bytes / per / 1e9, 4), "unit": "GB/s", "cores": int(blas_threads),
            "kind": "oracle", "seconds_per_step": round(per, 3),
            "host": {"os_cpu_count": os.cpu_count(), "affinity_cpus": affinity,
                     "torch_threads": torch.get_num_threads(), "blas_threads": int(blas_threads)},
            "sample": f"{len(picked)} of {w.num_seqs} sequences ({int(ws.seq_lens.sum())} tokens): oracle append "
                      f"of their new tokens + attention, {reps} reps; value = their cache bytes / time"}


if __name__ == "__main__":
    main()
