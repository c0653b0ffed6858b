/*
 * nvfp4kv_probe — measurement aid of the nvfp4kv benchmark (libnvfp4kv_probe.so).
 *
 * Not an operation of the NVFP4 KV cache: it gives the HBM read rate a plain
 * kernel reaches on the same device and the same number of bytes, the
 * ceiling against which the attention kernels' cache-read stream is judged.
 */
#ifndef NVFP4KV_PROBE_H
#define NVFP4KV_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Read `bytes` bytes at device pointer `data` (16-byte aligned, bytes a
 * positive multiple of 16) with `grid` workgroups of 256 lanes, 16 bytes per
 * lane and load, and write one XOR fold per wave to `sink` (device, at least
 * grid * 16 bytes, 4-byte aligned). Asynchronous on `stream`. Returns 0, 1
 * for a bad argument (nothing launched) or 4 if the launch failed.
 */
int32_t nvfp4kv_probe_read_stream(const void* data, int64_t bytes, int32_t grid, void* sink, int64_t sink_bytes,
                                  void* stream);

/*
 * Read every page a paged-attention decode batch reads, as a plain gather:
 * for each sequence b (seq_lens[b] keys, pages block_table[b *
 * max_blocks + p] for p < ceil(seq_lens[b] / block_size)) and each kv head,
 * the page's K slab and V slab, slab_bytes contiguous bytes each at pool +
 * id * stride_block + kv * stride_kv + head * stride_head (a page's rows
 * must be contiguous: row stride = row bytes, slab_bytes = block_size * row
 * bytes, a multiple of 16, at most 4096). Each sequence's pages are cut into
 * `splits` equal ranges, one workgroup of 256 lanes per (sequence, kv head,
 * range): num_seqs * num_kv_heads * splits workgroups. Block ids are clamped
 * to [0, num_blocks). One XOR fold per wave goes to sink (at least 16 bytes
 * per workgroup). Returns 0, 1 for a bad argument (nothing launched) or 4
 * if the launch failed.
 */
int32_t nvfp4kv_probe_read_pages(const void* pool, int64_t num_blocks, int64_t stride_block, int64_t stride_kv,
                                 int64_t stride_head, int32_t slab_bytes, int32_t block_size, int32_t num_kv_heads,
                                 const int32_t* block_table, int32_t max_blocks, const int32_t* seq_lens,
                                 int32_t num_seqs, int32_t splits, void* sink, int64_t sink_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4KV_PROBE_H */
